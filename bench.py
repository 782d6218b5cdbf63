"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME[,NAME...]] [--no-cpu-baseline]

One step runs the whole path over every workload's synthetic bf16 inputs (already
resident in HBM) -- by default both head-dim-128 workloads of the metric, B4 H16
N2048 (non-causal and causal) and B2 H16 N8192 (causal): for each workload and
mask, the forward, the 5-GEMM backward (preprocess with dq zeroing, dK/dV kernel
with fp32-atomic dQ) and the 7-GEMM backward (dQ kernel computing delta itself,
then the dK/dV kernel reading it).  Every kernel is bracketed by HIP events on the stream it runs on; W
untimed steps are followed by exactly K timed steps between two device
synchronisations.

Work accounting (masked tiles are not credited; pairs = unmasked score
elements): forward 4 d pairs, backward 10 d pairs for either design (the
5-GEMM count, as the 5-vs-7 comparison in "Potential algorithmic improvements
for backward pass" is made); the 7-GEMM design issues 14 d pairs.  `value` is
the step's credited TFLOP/s; one JSON line is printed at the end.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOPS and % of bf16 MFMA peak, hdim 128 N=2k-8k"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
KERNEL_SOURCES = {"fwd": "fa_fwd.hip", "dkdv": "fa_bwd.hip", "dkdv_atomic": "fa_bwd.hip", "dq": "fa_bwd.hip",
                  "preprocess": "fa_bwd.hip"}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in sorted({KERNEL_SOURCES[kernel], "fa_device.h"}):
        with open(os.path.join(ROOT, "exact_attention_102_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_flops(kernel: str, d: int, pairs: int) -> int:
    """Algorithmic MFMA flops of one launch: 2 d flops per pair per GEMM."""
    gemms = {"fwd": 2, "dkdv": 4, "dkdv_atomic": 5, "dq": 3}[kernel]
    return 2 * gemms * d * pairs


def preprocess_bytes(rows: int, d: int, zero_dq: bool) -> int:
    """Compulsory HBM bytes of the preprocess kernel: O fp32 + dO bf16 read, delta (+ dq zeros) written."""
    return rows * (4 * d + 2 * d + 4 + (4 * d if zero_dq else 0))


def stored_traffic(kernel: str, mask: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or None when the
    kernel's source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    ent = rec.get("kernels", {}).get("%s_%s" % (kernel, mask))
    if not ent or ent.get("source_hash") != source_hash(kernel):
        return None
    return ent.get("bytes_per_launch")


def atomic_adds_per_launch(B, H, N, d, causal, bk, bq):
    """fp32 atomic adds one launch of the fused dK/dV + dQ kernel issues: for each (key tile, visited
    query tile) pair, one add per dq element of the query tile's rows inside the sequence."""
    nkt, nqt = -(-N // bk), -(-N // bq)
    rows = 0
    for kt in range(nkt):
        q_first = (kt * bk) // bq if causal else 0
        for qt in range(q_first, nqt):
            rows += min(N, (qt + 1) * bq) - qt * bq
    return B * H * rows * d


def atomic_ceiling(d):
    """fp32 atomics per second that the committed probe summary measured for the default atomic pattern at head
    dim d (buffer atomics, no cache-policy bits, key tiles of a head on one XCD), or None."""
    path = os.path.join(ROOT, "profiles", "atomic_dq_probe.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if not line.startswith("{"):
                continue
            rec = json.loads(line)
            if rec.get("probe") == "buffer aux=0" and rec.get("mapping") == "xcd" and rec["d"] == d:
                return rec["G_per_s"]
    return None


def cpu_baseline(cases, heads_per_workload=-1):
    """The fp64 oracle as it stands, timed on this host's cores over the step's cases (every head of each
    workload, or the first `heads_per_workload`)."""
    from threadpoolctl import threadpool_limits

    import oracle
    import workloads
    from exact_attention_102_amd.flops import attention_flops

    cores = oracle.usable_cores()
    flops, parts, used = 0, [], 1
    host = {}
    for case in cases:
        if case.w.name not in host:
            host[case.w.name] = [workloads.bf16_to_f64(workloads.to_bf16(x)) for x in workloads.draw_workload(case.w)]
    t0 = time.perf_counter()
    for case in cases:
        w = case.w
        nh = w.B * w.H if heads_per_workload < 0 else min(heads_per_workload, w.B * w.H)
        heads = list(range(nh))
        workers = max(1, min(cores, len(heads)))
        blas = max(1, cores // workers)
        used = max(used, workers * blas)
        q, k, v, do = host[w.name]
        with threadpool_limits(limits=blas, user_api="blas"):
            oracle.attention_forward_batched(q, k, v, w.scale, case.causal, workers=workers, heads=heads)
            oracle.attention_backward_batched(q, k, v, do, w.scale, case.causal, workers=workers, heads=heads)
        f = attention_flops(1, len(heads), w.N, w.d, case.causal)
        flops += f["fwd"] + f["bwd_effective"]
        parts.append("%d of %d heads of %s" % (len(heads), w.B * w.H, case.key))
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": used, "kind": "oracle",
            "sample": "%s; fwd+bwd in fp64 numpy, %.1f s wall" % ("; ".join(parts), dt)}


DEFAULT_WORKLOADS = "b4_h16_n2048_d128,b2_h16_n8192_d128_causal"
KERNELS = ["fwd", "preprocess5", "dkdv_atomic", "dq", "dkdv"]


class Case:
    """One (workload, mask) of the step: its device inputs and outputs."""

    def __init__(self, w, causal, dev_inputs):
        import torch
        self.w, self.causal = w, causal
        self.mask = "causal" if causal else "full"
        self.key = "%s/%s" % (w.name, self.mask)
        B, H, N, d = w.B, w.H, w.N, w.d
        self.q, self.k, self.v, self.do = dev_inputs
        f32 = dict(dtype=torch.float32, device=self.q.device)
        self.o = torch.empty((B, H, N, d), **f32)
        self.lse = torch.empty((B, H, N), **f32)
        self.delta = torch.empty((B, H, N), **f32)
        self.delta7 = torch.empty((B, H, N), **f32)
        self.dq5, self.dk5, self.dv5 = (torch.empty((B, H, N, d), **f32) for _ in range(3))
        self.dq7, self.dk7, self.dv7 = (torch.empty((B, H, N, d), **f32) for _ in range(3))

    def run(self, stream, ev):
        """fwd | preprocess5 | dkdv_atomic | dq (+ delta) | dkdv, events ev[0..5] around them."""
        from exact_attention_102_amd import fa_bwd_dkdv, fa_bwd_dq_delta, fa_bwd_preprocess, fa_fwd
        w, c = self.w, self.causal
        if ev:
            ev[0].record(stream)
        fa_fwd(self.q, self.k, self.v, c, w.scale, o=self.o, lse=self.lse, stream=stream)
        if ev:
            ev[1].record(stream)
        fa_bwd_preprocess(self.o, self.do, delta=self.delta, dq=self.dq5, stream=stream)
        if ev:
            ev[2].record(stream)
        fa_bwd_dkdv(self.q, self.k, self.v, self.do, self.lse, self.delta, c, w.scale, True, self.dk5, self.dv5,
                    dq=self.dq5, stream=stream)
        if ev:
            ev[3].record(stream)
        fa_bwd_dq_delta(self.q, self.k, self.v, self.o, self.do, self.lse, c, w.scale, self.delta7, self.dq7,
                        stream=stream)
        if ev:
            ev[4].record(stream)
        fa_bwd_dkdv(self.q, self.k, self.v, self.do, self.lse, self.delta7, c, w.scale, False, self.dk7, self.dv7,
                    stream=stream)
        if ev:
            ev[5].record(stream)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOADS,
                    help="comma-separated workload names (workloads.WORKLOADS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=-1, help="heads per workload in the oracle sample (-1: all)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only (attention heads would shard across GPUs with no exchange; "
              "no multi-GPU run is provided). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads
    from exact_attention_102_amd import fa_config_name, fa_default_config, lib
    from exact_attention_102_amd.flops import attention_flops, mfa_op_counts

    lib()  # fail loudly if libfa.so is missing
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    wls = [workloads.WORKLOADS[n] for n in args.workload.split(",") if n]
    cases = []
    for w in wls:
        log("workload %s B=%d H=%d N=%d d=%d" % (w.name, w.B, w.H, w.N, w.d))
        dev = tuple(workloads.to_bf16(x).cuda() for x in workloads.draw_workload(w))
        for causal in ([False, True] if not w.causal else [True]):
            cases.append(Case(w, causal, dev))
    stream = torch.cuda.current_stream()

    def step(record):
        for ci, case in enumerate(cases):
            case.run(stream, record[ci] if record is not None else None)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    events = [[[torch.cuda.Event(enable_timing=True) for _ in range(len(KERNELS) + 1)] for _ in cases] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per (case, kernel) mean duration in ms over the K timed steps
    dur = {}
    for ci, case in enumerate(cases):
        for ki, kn in enumerate(KERNELS):
            ts = [events[s][ci][ki].elapsed_time(events[s][ci][ki + 1]) for s in range(args.steps)]
            dur[(case.key, kn)] = sum(ts) / len(ts)

    total_flops = 0
    passes = {}
    best = None
    for case in cases:
        w = case.w
        fl = attention_flops(w.B, w.H, w.N, w.d, case.causal)
        p = fl["pairs"]
        t_fwd = dur[(case.key, "fwd")]
        t_b5 = dur[(case.key, "preprocess5")] + dur[(case.key, "dkdv_atomic")]
        t_b7 = dur[(case.key, "dq")] + dur[(case.key, "dkdv")]
        total_flops += fl["fwd"] + 2 * fl["bwd_effective"]
        ent = {
            "fwd_tflops": fl["fwd"] / t_fwd / 1e9, "fwd_ms": t_fwd,
            "bwd_5gemm_tflops": fl["bwd_effective"] / t_b5 / 1e9, "bwd_5gemm_ms": t_b5,
            "bwd_7gemm_tflops": fl["bwd_effective"] / t_b7 / 1e9, "bwd_7gemm_ms": t_b7,
            "bwd_7gemm_issued_tflops": fl["bwd_7gemm_issued"] / t_b7 / 1e9,
            "kernel_ms": {kn: round(dur[(case.key, kn)], 4) for kn in KERNELS},
            "pairs": p,
            "mfa_op_counts_per_dispatch": mfa_op_counts(w.N, w.d),
        }
        for key in ("fwd", "bwd_5gemm", "bwd_7gemm"):
            ent[key + "_pct_peak"] = 100.0 * ent[key + "_tflops"] / PEAK_BF16_TFLOPS
        ent["faster_bwd"] = "5gemm" if t_b5 <= t_b7 else "7gemm"
        ent["t7_over_t5"] = t_b7 / t_b5
        passes[case.key] = ent
        # the dominant kernel: the one that takes the most time per step
        for kn in ("fwd", "dkdv_atomic", "dkdv", "dq"):
            t = dur[(case.key, kn)]
            if best is None or t > best[2]:
                best = (kn, case, t, kernel_flops(kn, w.d, p))

    kn, case, t_ms, kflops = best
    w = case.w
    achieved = kflops / (t_ms * 1e-3) / 1e12
    traffic = stored_traffic(kn, case.mask, w.name)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": "%s (%s, %s mask)" % (kn, w.name, case.mask), "launch_ms": round(t_ms, 4),
                "flops_per_launch": kflops}
    if kn == "dkdv_atomic":
        # the fused dQ atomics, not only the MFMAs, bound this kernel: their rate against the probe's ceiling
        from exact_attention_102_amd.report import tile_shape
        bk, bq = tile_shape(fa_config_name(2, w.d, case.causal, fa_default_config(2, w.d, case.causal)))
        adds = atomic_adds_per_launch(w.B, w.H, w.N, w.d, case.causal, bk, bq)
        rate = adds / (t_ms * 1e-3) / 1e9
        ceil = atomic_ceiling(w.d)
        roofline["atomics"] = {"adds_per_launch": adds, "achieved_G_per_s": round(rate, 1),
                               "probe_ceiling_G_per_s": ceil,
                               "frac": round(rate / ceil, 4) if ceil else None}
    value = total_flops / (ms_per_step * 1e-3) / 1e12

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle")
        cpu = cpu_baseline(cases, args.cpu_heads)

    tiles = {}
    for wd in sorted({w.d for w in wls}):
        for causal in (False, True):
            m = "causal" if causal else "full"
            tiles["d%d_%s" % (wd, m)] = {
                "fwd": fa_config_name(0, wd, causal, fa_default_config(0, wd, causal)),
                "dkdv": fa_config_name(1, wd, causal, fa_default_config(1, wd, causal)),
                "dkdv_atomic": fa_config_name(2, wd, causal, fa_default_config(2, wd, causal)),
                "dq": fa_config_name(3, wd, causal, fa_default_config(3, wd, causal))}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": " + ".join(c.key for c in cases),
                   "workloads": [{"name": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "scale": w.scale}
                                 for w in wls],
                   "step": "per workload and mask: fwd + 5-GEMM bwd + 7-GEMM bwd", "tiles": tiles},
        "passes": {m: {k2: (round(v2, 4) if isinstance(v2, float) else v2) for k2, v2 in p.items()}
                   for m, p in passes.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
