"""Head-dimension spectrum: throughput of the forward and both backward designs
across the 42 head dimensions of the sweep in "Potential algorithmic improvements
for backward pass" (4..96 step 4, ..160 step 8, ..256 step 16, ..384 step 32).

    python -m exact_attention_102_amd.dspectrum [--B 4 --H 16 --N 2048] [--out profiles/dspectrum_b4_h16_n2048.md]

Each point runs the general entry points on seeded N(0,1) bf16 inputs (the first D
columns of one draw), non-causal: head dims other than the built 64/96/128/192/256
and 288/320/352/384 run on the kernels of the next built size, padded inside the kernels when D is a
multiple of 8 and through zero-padded copies otherwise,
with that page's protocol: 5 trials of 5 back-to-back dispatches, best trial.  It
reports TFLOP/s credited with the true head dim (4D flop per pair forward, 10D for
both backward designs), the page's instruction rates ((2D+5) N^2 forward, (3D+5)
N^2 + (4D+5) N^2 for the backward kernels, in G per second), and which backward
design is faster -- the page expects the answer to depend on head dim and chip.
Above 256 the dK/dV accumulators of all columns no longer fit the register file, so
the dK/dV pass runs one 128-column window per workgroup and recomputes S and dP for
each window (three windows at 384); the forward holds Q and O for all columns.
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
BUILT = (64, 96, 128, 192, 256, 288, 320, 352, 384)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--B", type=int, default=4)
    ap.add_argument("--H", type=int, default=16)
    ap.add_argument("--N", type=int, default=2048)
    ap.add_argument("--seed", type=int, default=11)
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    import torch

    import workloads
    from exact_attention_102_amd import (FA_BWD_5GEMM_ATOMIC, FA_BWD_7GEMM, fa_bwd_general,
                                         fa_bwd_general_workspace_size, fa_fwd_general,
                                         fa_fwd_general_workspace_size, lib)
    from exact_attention_102_amd.flops import attention_flops, d_spectrum
    from exact_attention_102_amd.sweep import time_calls

    lib()
    if not torch.cuda.is_available():
        raise SystemExit("dspectrum needs a GPU")
    B, H, N = args.B, args.H, args.N
    # one seeded draw at the widest built head dim; each point uses its first D columns
    full = [workloads.to_bf16(x).cuda() for x in workloads.draw(B, H, N, BUILT[-1], args.seed)]
    rows = []
    for D in d_spectrum():
        rec = {"D": D, "B": B, "H": H, "N": N}
        if D > BUILT[-1]:
            rec["supported"] = False
            rows.append(rec)
            print(json.dumps(rec), flush=True)
            continue
        scale = D ** -0.5
        q, k, v, do = (x[..., :D].contiguous() for x in full)
        dev = q.device
        o = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = (torch.empty((B, H, N, D), dtype=torch.float32, device=dev) for _ in range(3))
        wsf = torch.empty(max(fa_fwd_general_workspace_size(B, H, N, D), 16), dtype=torch.uint8, device=dev)
        wsb = torch.empty(max(fa_bwd_general_workspace_size(B, H, N, D, FA_BWD_7GEMM), 16), dtype=torch.uint8,
                          device=dev)

        def fwd():
            fa_fwd_general(q, k, v, False, scale, o=o, lse=lse, workspace=wsf)

        def bwd(var):
            return lambda: fa_bwd_general(q, k, v, o, lse, do, False, scale, var, dq=dq, dk=dk, dv=dv, workspace=wsb)

        fwd()
        torch.cuda.synchronize()
        fl = attention_flops(B, H, N, D, False)
        n2 = B * H * N * N
        t_f, _ = time_calls(fwd, torch)
        t_5, _ = time_calls(bwd(FA_BWD_5GEMM_ATOMIC), torch)
        t_7, _ = time_calls(bwd(FA_BWD_7GEMM), torch)
        rec.update({
            "supported": True, "padded_to": min(b for b in BUILT if b >= D),
            "fwd_ms": round(t_f, 4), "bwd5_ms": round(t_5, 4), "bwd7_ms": round(t_7, 4),
            "fwd_tflops": round(fl["fwd"] / t_f / 1e9, 1),
            "bwd5_tflops": round(fl["bwd_effective"] / t_5 / 1e9, 1),
            "bwd7_tflops": round(fl["bwd_effective"] / t_7 / 1e9, 1),
            "fwd_ginstrs": round((2 * D + 5) * n2 / t_f / 1e6, 0),
            "bwd7_ginstrs": round(((3 * D + 5) + (4 * D + 5)) * n2 / t_7 / 1e6, 0),
            "t7_over_t5": round(t_7 / t_5, 3),
        })
        rows.append(rec)
        print(json.dumps(rec), flush=True)
        del q, k, v, do, o, lse, dq, dk, dv, wsf, wsb
        torch.cuda.empty_cache()

    if args.out:
        with open(args.out, "w") as fh:
            fh.write("# Head-dimension spectrum (one MI355X), B%d H%d N%d, non-causal\n\n" % (B, H, N))
            # the command as run from the repository root, writing the committed file
            fh.write("Command (from the repository root): `python -m exact_attention_102_amd.dspectrum --out "
                     "profiles/%s`\n\n" % os.path.basename(args.out))
            fh.write("Best of 5 trials x 5 dispatches.  TFLOP/s credit the true head dim D: 4D (fwd) and 10D (both "
                     "backward designs) flop per pair, peak 2500.  G instr/s: the page's (2D+5) N^2 for the forward "
                     "and (3D+5) N^2 + (4D+5) N^2 for the 7-GEMM backward's two kernels.  Head dims other than "
                     "64/96/128/192/256/288/320/352/384 run on the kernels of the next built size (`padded`): padded inside the kernels "
                     "when D is a multiple of 8, through zero-padded copies otherwise.\n\n")
            fh.write("| D | padded | fwd TF | 5-GEMM bwd TF | 7-GEMM bwd TF | fwd G instr/s | 7-GEMM bwd G instr/s | "
                     "t7/t5 | faster bwd |\n|---|---|---|---|---|---|---|---|---|\n")
            for r in rows:
                if not r["supported"]:
                    fh.write("| %d | not built | - | - | - | - | - | - | - |\n" % r["D"])
                    continue
                fh.write("| %d | %d | %.1f | %.1f | %.1f | %.0f | %.0f | %.3f | %s |\n" % (
                    r["D"], r["padded_to"], r["fwd_tflops"], r["bwd5_tflops"], r["bwd7_tflops"], r["fwd_ginstrs"],
                    r["bwd7_ginstrs"], r["t7_over_t5"], "7-GEMM" if r["t7_over_t5"] < 1 else "5-GEMM"))


if __name__ == "__main__":
    main()
