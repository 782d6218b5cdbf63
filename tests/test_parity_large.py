"""GPU parity at the largest sequence lengths (one head each, both masks, both backward
designs), where the oracle cannot compute whole tensors in seconds.

* Sampled query rows against the fp64 oracle, at the fixed-shape bar: O (max-abs
  1e-2), LSE (max-abs 1e-3) and dQ (relative L2 2e-2 over the sampled rows).  Each is
  a function of its own row: under the causal mask query i attends to keys 0..i, so
  the oracle runs the row against that key prefix without a mask.
* Sampled key rows of dK and dV, element by element against the oracle's key-row
  backward (every query row that attends to a sampled key, each with its full-row
  softmax).  Under the causal mask the sampled keys sit near the end, where few query
  rows attend to them, so the oracle finishes in seconds at every length; without the
  mask every query row attends to every key, so the non-causal sampled-key case runs
  at N = 65536, d = 64 (about a teraflop of fp64 work).  Bar: relative L2 2e-2 over
  the sampled rows and the per-row bound of parity_util.
* dK and dV through identities of the exact gradients that hold at any size, checked
  on the whole tensors: every row of dS sums to zero, so sum_j dK_j = 0; <Q, dQ> =
  <K, dK> (both are scale * sum dS * S); and, without the mask, sum_j dV_j =
  sum_i dO_i (the rows of P sum to one).  Tolerances 2e-2 relative to the norms of
  the summed terms.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from parity_util import (GRAD_REL_L2, LSE_MAX_ABS, O_MAX_ABS, ROW_REL, VARIANTS, gpu_backward, gpu_forward,
                         make_inputs, note, rel_l2, row_errors)

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

REL = 2e-2


@pytest.mark.parametrize("N,d", [(131072, 128), (65536, 256), (262144, 64), (32768, 384)], ids=lambda x: str(x))
@pytest.mark.parametrize("causal", [False, True])
def test_longest_sequences(N, d, causal):
    B, H = 1, 1
    scale = 1.0 / math.sqrt(d)
    note("large N=%d d=%d causal=%d" % (N, d, causal))
    dev, host, _ = make_inputs(B, H, N, d, seed=4000 + d)
    q, k, v, do = (x[0, 0] for x in host)
    rows = sorted({0, 1, 777, N // 2 + 3, N - 2, N - 1})
    o, lse = gpu_forward(dev, causal, scale)
    o_s = o[0, 0, rows].cpu().numpy()
    l_s = lse[0, 0, rows].cpu().numpy()
    refs = []
    for a, i in enumerate(rows):
        keys = slice(0, i + 1) if causal else slice(0, N)
        ro, rl = oracle.attention_forward(q[i:i + 1], k[keys], v[keys], scale, False)
        gq, _, _ = oracle.attention_backward(q[i:i + 1], k[keys], v[keys], do[i:i + 1], scale, False)
        assert np.max(np.abs(o_s[a] - ro[0])) <= O_MAX_ABS
        assert abs(l_s[a] - rl[0]) <= LSE_MAX_ABS
        refs.append(gq[0])
    refs = np.stack(refs)
    keys = [N - 1, N - 2, N - 37, N - 300, N - 1000] if causal else None
    if causal:
        rk, rv = oracle.attention_backward_key_rows(q, k, v, do, scale, True, keys)
    qd, kd, dod = (x[0, 0].double() for x in (dev[0], dev[1], dev[3]))
    for name, var in VARIANTS.items():
        note("  bwd %s" % name)
        dq, dk, dv = gpu_backward(dev, o, lse, causal, scale, var)
        assert np.all(np.isfinite(dq[0, 0, rows].cpu().numpy()))
        e = rel_l2(dq[0, 0, rows].cpu().numpy(), refs)
        assert e <= GRAD_REL_L2, "%s sampled dQ rel-L2 %.3e" % (name, e)
        if causal:
            check_key_rows(name, dk[0, 0, keys].cpu().numpy(), dv[0, 0, keys].cpu().numpy(), rk, rv)
        dq64, dk64, dv64 = (t[0, 0].double() for t in (dq, dk, dv))
        assert torch.isfinite(dk64).all() and torch.isfinite(dv64).all()
        # sum_j dK_j = 0, relative to the size of the terms summed
        s = torch.linalg.norm(dk64.sum(dim=0)) / torch.linalg.norm(dk64)
        assert s <= REL, "%s: |sum_j dK_j| / |dK| = %.3e" % (name, s)
        a_, b_ = float((qd * dq64).sum()), float((kd * dk64).sum())
        ref = float(torch.linalg.norm(qd) * torch.linalg.norm(dq64))
        assert abs(a_ - b_) <= REL * ref, "%s: <Q,dQ> %.6e vs <K,dK> %.6e" % (name, a_, b_)
        if not causal:
            sv, so = dv64.sum(dim=0), dod.sum(dim=0)
            e = float(torch.linalg.norm(sv - so) / torch.linalg.norm(dod))
            assert e <= REL, "%s: |sum dV - sum dO| / |dO| = %.3e" % (name, e)
        del dq, dk, dv
    del o, lse
    torch.cuda.empty_cache()


def check_key_rows(name, dk, dv, rk, rv):
    for what, g, r in (("dK", dk, rk), ("dV", dv, rv)):
        assert np.all(np.isfinite(g)), "%s sampled %s not finite" % (name, what)
        e = rel_l2(g, r)
        worst, own = row_errors(g, r)
        note("  %s sampled %s rows: rel-L2 %.2e, worst row %.2e of RMS (%.2e of own norm)" % (name, what, e, worst,
                                                                                            own))
        assert e <= GRAD_REL_L2, "%s sampled %s rel-L2 %.3e" % (name, what, e)
        assert worst <= ROW_REL, "%s sampled %s worst row %.3e" % (name, what, worst)


def test_sampled_key_rows_without_mask():
    """Non-causal: every query row attends to every key, so the oracle's key-row backward
    runs all N rows (about 1.1 TFLOP of fp64 at N = 65536, d = 64)."""
    B, H, N, d = 1, 1, 65536, 64
    scale = 1.0 / math.sqrt(d)
    note("large non-causal key rows N=%d d=%d" % (N, d))
    dev, host, _ = make_inputs(B, H, N, d, seed=4100)
    q, k, v, do = (x[0, 0] for x in host)
    keys = [0, 1, 4095, N // 2 + 5, N - 1]
    rk, rv = oracle.attention_backward_key_rows(q, k, v, do, scale, False, keys)
    o, lse = gpu_forward(dev, False, scale)
    for name, var in VARIANTS.items():
        dq, dk, dv = gpu_backward(dev, o, lse, False, scale, var)
        check_key_rows(name, dk[0, 0, keys].cpu().numpy(), dv[0, 0, keys].cpu().numpy(), rk, rv)
        del dq, dk, dv
