"""HBM traffic per kernel launch from rocprofv3 counters.

Two steps, each a command that runs committed files only:

  1. Under the profiler (one counter per run; R = the repository root):
       rocprofv3 --pmc FETCH_SIZE -d <dir_fetch> -o run --output-format csv -- \\
           python3 $R/exact_attention_102_amd/traffic.py --run --workload b4_h16_n2048_d128
       rocprofv3 --pmc WRITE_SIZE -d <dir_write> -o run --output-format csv -- \\
           python3 $R/exact_attention_102_amd/traffic.py --run --workload b4_h16_n2048_d128
     --run performs a device copy of a known size (calibration) and then one launch of
     every kernel of the path (forward, preprocess, dK/dV, dK/dV with atomic dQ, dQ)
     for each mask of the workload.
  2. Summarise:
       python3 exact_attention_102_amd/traffic.py --parse <dir_fetch> <dir_write> \\
           --workload b4_h16_n2048_d128 --out profiles/traffic_b4_h16_n2048_d128.json

FETCH_SIZE / WRITE_SIZE are reported in KiB per dispatch.  The copy kernel moves
exactly COPY_BYTES in each direction, so bytes = counter * 1024 * (COPY_BYTES /
(copy counter * 1024)); the factor is recorded.  Each kernel's entry carries the
hash of the sources it was built from, so bench.py reports the stored traffic only
while the kernel is unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

COPY_BYTES = 512 * 1024 * 1024
SOURCES = {"fwd": "fa_fwd.hip", "dkdv": "fa_bwd.hip", "dkdv_atomic": "fa_bwd.hip", "dq": "fa_bwd.hip",
           "preprocess": "fa_bwd.hip"}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in sorted({SOURCES[kernel], "fa_device.h"}):
        with open(os.path.join(ROOT, "exact_attention_102_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def run(workload: str):
    import torch

    import workloads
    from exact_attention_102_amd import fa_bwd_dkdv, fa_bwd_dq_delta, fa_bwd_preprocess, fa_fwd

    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    w = workloads.WORKLOADS[workload]
    B, H, N, d = w.B, w.H, w.N, w.d
    q, k, v, do = (workloads.to_bf16(x).cuda() for x in workloads.draw_workload(w))
    f32 = dict(dtype=torch.float32, device="cuda")
    o = torch.empty((B, H, N, d), **f32)
    lse = torch.empty((B, H, N), **f32)
    delta = torch.empty((B, H, N), **f32)
    dq, dk, dv = (torch.empty((B, H, N, d), **f32) for _ in range(3))
    for causal in ([False, True] if not w.causal else [True]):
        fa_fwd(q, k, v, causal, w.scale, o=o, lse=lse)
        fa_bwd_preprocess(o, do, delta=delta, dq=dq)
        fa_bwd_dkdv(q, k, v, do, lse, delta, causal, w.scale, True, dk, dv, dq=dq)
        fa_bwd_dq_delta(q, k, v, o, do, lse, causal, w.scale, delta, dq)
        fa_bwd_dkdv(q, k, v, do, lse, delta, causal, w.scale, False, dk, dv)
        torch.cuda.synchronize()
    print("traffic run done", flush=True)


def classify(name: str):
    """(kernel key, mask) of a profiled kernel name, or None."""
    m = re.search(r"fa::(\w+)_kernel<([^>]*)>", name)
    if not m:
        return None
    kind, targs = m.group(1), [t.strip() for t in m.group(2).split(",")]
    # template arguments: fwd <D, DV, tile, waves, occupancy, CAUSAL, DROP, OPT>; dq <D, DV, tile, waves,
    # occupancy, CAUSAL, DROP>; dkdv <D, DV, BQ, waves, CAUSAL, ATOMIC, KV_LDS, DEFER, DROP>;
    # dkdv_wide <D, DV, BQ, waves, CAUSAL, ATOMIC>; dkdv_split <D, DV, window, BQ, waves, CAUSAL, ATOMIC>;
    # dropout kernels are not classified
    flag = lambda i: i < len(targs) and targs[i] == "true"  # noqa: E731
    if (kind in ("fwd", "dq") and flag(6)) or (kind == "dkdv" and flag(8)):
        return None
    if kind in ("dkdv_wide", "dkdv"):
        causal, atomic = flag(4), flag(5)
        return ("dkdv_atomic" if atomic else "dkdv"), ("causal" if causal else "full")
    if kind == "dkdv_split":
        causal, atomic = flag(5), flag(6)
        return ("dkdv_atomic" if atomic else "dkdv"), ("causal" if causal else "full")
    if kind in ("fwd", "dq"):
        return kind, ("causal" if flag(5) else "full")
    if kind == "preprocess":
        return "preprocess", None
    return None


def read_counter(dirname: str, counter: str):
    """[(kernel name, value KiB)] in dispatch order from a rocprofv3 counter_collection csv."""
    files = glob.glob(os.path.join(dirname, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError("no counter_collection.csv under " + dirname)
    rows = []
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if r.get("Counter_Name") != counter:
                continue
            rows.append((int(r.get("Dispatch_Id", 0)), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    # one value per dispatch (rocprofv3 may emit one row per dispatch already aggregated)
    agg = {}
    for disp, name, val in rows:
        agg.setdefault(disp, [name, 0.0])
        agg[disp][1] += val
    return [(agg[k][0], agg[k][1]) for k in sorted(agg)]


def parse(fetch_dir: str, write_dir: str, workload: str, out: str):
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    copy_f = [v for n, v in fetch if "copy" in n.lower() or "elementwise" in n.lower()]
    copy_w = [v for n, v in write if "copy" in n.lower() or "elementwise" in n.lower()]
    # the copy is the largest-traffic non-attention dispatch
    cf = COPY_BYTES / (max(copy_f) * 1024.0)
    cw = COPY_BYTES / (max(copy_w) * 1024.0)
    res = {"workload": workload, "copy_bytes": COPY_BYTES, "fetch_calibration": cf, "write_calibration": cw,
           "kernels": {}}
    for (nf, vf), (nw, vw) in zip(fetch, write):
        c = classify(nf)
        if c is None or c[0] == "preprocess":
            continue
        key = "%s_%s" % c
        res["kernels"][key] = {"name": nf, "fetch_bytes": vf * 1024 * cf, "write_bytes": vw * 1024 * cw,
                               "bytes_per_launch": vf * 1024 * cf + vw * 1024 * cw,
                               "source_hash": source_hash(c[0])}
    with open(out, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--run", action="store_true")
    ap.add_argument("--parse", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--workload", default="b4_h16_n2048_d128")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()
    if a.run:
        run(a.workload)
    if a.parse:
        parse(a.parse[0], a.parse[1], a.workload, a.out or os.path.join(ROOT, "profiles", "traffic_%s.json" % a.workload))


if __name__ == "__main__":
    main()
