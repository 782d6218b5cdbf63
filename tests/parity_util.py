"""Helpers for the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same seeded bf16 inputs, and compare at the stated bar.

Tolerances (bf16 inputs, fp32 accumulation): O max-abs <= 1e-2, LSE max-abs
<= 1e-3, dQ/dK/dV relative L2 <= 2e-2 (relative to the oracle's norm).  Beside the
whole-tensor figure every gradient comparison also bounds the worst single row:
the largest per-row error norm may be at most ROW_REL of the root-mean-square row
norm, so an error confined to a few rows (which the whole-tensor norm dilutes) still
fails; the largest error relative to a row's own norm is reported.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads
from exact_attention_102_amd import FA_BWD_5GEMM_ATOMIC, FA_BWD_7GEMM, fa_bwd, fa_fwd

O_MAX_ABS = 1e-2
LSE_MAX_ABS = 1e-3
GRAD_REL_L2 = 2e-2
ZERO_GRAD_ABS = 1e-5
ROW_REL = 5e-2


def note(msg: str):
    print("[parity] " + msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64))))


def make_inputs(B, H, N, d, seed, qk_mult=1.0):
    q, k, v, do = workloads.draw(B, H, N, d, seed, qk_mult)
    bf = [workloads.to_bf16(x) for x in (q, k, v, do)]
    host64 = [workloads.bf16_to_f64(x) for x in bf]
    dev = [x.cuda() for x in bf]
    return dev, host64, (q, k, v, do)


def gpu_forward(dev, causal, scale, cfg=-1):
    q, k, v, _ = dev
    o, lse = fa_fwd(q, k, v, causal, scale, cfg=cfg)
    torch.cuda.synchronize()
    return o, lse


def gpu_backward(dev, o, lse, causal, scale, variant, cfg_dkdv=-1, cfg_dq=-1):
    q, k, v, do = dev
    dq, dk, dv = fa_bwd(q, k, v, o, lse, do, causal, scale, variant, cfg_dkdv=cfg_dkdv, cfg_dq=cfg_dq)
    torch.cuda.synchronize()
    return dq, dk, dv


def check_forward(o, lse, ref_o, ref_lse, heads=None):
    o = o.cpu().numpy().reshape(-1, *o.shape[2:])
    lse = lse.cpu().numpy().reshape(-1, lse.shape[-1])
    ref_o = ref_o.reshape(-1, *ref_o.shape[2:])
    ref_lse = ref_lse.reshape(-1, ref_lse.shape[-1])
    if heads is not None:
        o, lse, ref_o, ref_lse = o[heads], lse[heads], ref_o[heads], ref_lse[heads]
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    eo, el = max_abs(o, ref_o), max_abs(lse, ref_lse)
    assert eo <= O_MAX_ABS, "O max-abs error %.3e > %.0e" % (eo, O_MAX_ABS)
    assert el <= LSE_MAX_ABS, "LSE max-abs error %.3e > %.0e" % (el, LSE_MAX_ABS)
    return eo, el


def row_errors(g, r):
    """(worst row error / RMS row norm, worst row error / own row norm) over the rows of the last axis."""
    g = np.asarray(g, dtype=np.float64).reshape(-1, np.shape(g)[-1])
    r = np.asarray(r, dtype=np.float64).reshape(-1, np.shape(r)[-1])
    en = np.linalg.norm(g - r, axis=1)
    rn = np.linalg.norm(r, axis=1)
    rms = float(np.sqrt(np.mean(rn * rn)))
    big = rn > 1e-3 * rms
    own = float(np.max(en[big] / rn[big])) if np.any(big) else 0.0
    return float(np.max(en)) / max(rms, 1e-300), own


def check_backward(grads, refs, heads=None, label=""):
    errs = []
    rows = []
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        g = g.cpu().numpy() if hasattr(g, "cpu") else np.asarray(g)
        g = g.reshape(-1, *g.shape[2:])
        r = np.asarray(r).reshape(-1, *np.shape(r)[2:])
        if heads is not None:
            g, r = g[heads], r[heads]
        assert np.all(np.isfinite(g)), name + " has non-finite values"
        if not np.any(r):
            # The exact gradient is identically zero (e.g. N = 1: dS = P (dP - delta) = 0), where a relative
            # error is undefined; the kernel's value is then pure rounding of dP - delta and must be tiny.
            e = max_abs(g, r)
            assert e <= ZERO_GRAD_ABS, "%s should be ~0, max-abs %.3e" % (name, e)
        else:
            e = rel_l2(g, r)
            assert e <= GRAD_REL_L2, "%s rel-L2 error %.3e > %.0e" % (name, e, GRAD_REL_L2)
            worst, own = row_errors(g, r)
            assert worst <= ROW_REL, "%s worst row error %.3e of the RMS row norm > %.0e" % (name, worst, ROW_REL)
            rows.append("%s %.1e/%.1e" % (name, worst, own))
        errs.append(e)
    if rows:
        note("  %srel-L2 %s; worst row (vs RMS / own norm) %s" % (label, " ".join("%.1e" % x for x in errs),
                                                                   ", ".join(rows)))
    return errs


def oracle_forward(host64, scale, causal, heads=None):
    q, k, v, _ = host64
    return oracle.attention_forward_batched(q, k, v, scale, causal, heads=heads)


def oracle_backward(host64, scale, causal, heads=None):
    q, k, v, do = host64
    return oracle.attention_backward_batched(q, k, v, do, scale, causal, heads=heads)


VARIANTS = {"5gemm": FA_BWD_5GEMM_ATOMIC, "7gemm": FA_BWD_7GEMM}
