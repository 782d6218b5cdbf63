"""The no-allocation backward entry point (fa_bwd_noalloc) against fa_bwd, through the C ABI.

fa_bwd_noalloc runs the same kernels as fa_bwd with the library's fixed device scratch in
place of the caller's workspace, so on the same inputs its results must equal fa_bwd's:
bit for bit for everything computed without atomics (the 7-GEMM design's dQ, dK, dV and
the 5-GEMM design's dK, dV), and to the fp32 reordering of the atomic sum for the 5-GEMM
dQ.  Calls in a row, each smaller than the one before, check that the shared scratch carries
nothing over from the previous call.  The results are also held to the oracle's bar.
"""
import math

import numpy as np
import pytest
import torch

from parity_util import VARIANTS, check_backward, gpu_forward, make_inputs, note, oracle_backward, rel_l2

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

# each call smaller than the one before; the last runs the head-dim-384 kernels
CASES = [((2, 4, 1000, 128), True, 11), ((1, 2, 300, 64), False, 12), ((1, 1, 200, 384), True, 13)]


@pytest.mark.parametrize("variant", ["7gemm", "5gemm"])
def test_noalloc_matches_fa_bwd_on_two_calls(variant):
    from exact_attention_102_amd import fa_bwd, fa_bwd_noalloc
    for (B, H, N, d), causal, seed in CASES:
        note("noalloc %s B=%d H=%d N=%d d=%d causal=%d" % (variant, B, H, N, d, causal))
        scale = 1.0 / math.sqrt(d)
        dev, host, _ = make_inputs(B, H, N, d, seed=seed)
        o, lse = gpu_forward(dev, causal, scale)
        q, k, v, do = dev
        ref = fa_bwd(q, k, v, o, lse, do, causal, scale, VARIANTS[variant])
        outs = tuple(torch.full((B, H, N, d), float("nan"), dtype=torch.float32, device="cuda") for _ in range(3))
        got = fa_bwd_noalloc(q, k, v, o, lse, do, causal, scale, VARIANTS[variant], *outs)
        torch.cuda.synchronize()
        for name, g, r in zip(("dq", "dk", "dv"), got, ref):
            if variant == "5gemm" and name == "dq":
                e = rel_l2(g.cpu().numpy(), r.cpu().numpy())
                assert e <= 1e-5, "dq differs from fa_bwd's by rel-L2 %.3e" % e
            else:
                assert torch.equal(g, r), name + " differs from fa_bwd's"
        check_backward(got, oracle_backward(host, scale, causal))


def test_noalloc_rejects_sizes_beyond_its_scratch():
    from exact_attention_102_amd import FA_ERR_TOO_LARGE, FA_NOALLOC_MAX_ROWS, lib
    import ctypes
    P = ctypes.c_void_p(0x7f0000000000)   # never dereferenced: the size check comes first
    N = FA_NOALLOC_MAX_ROWS // 8 + 1       # B * H * N = 8 N > the maximum
    st = lib().fa_bwd_noalloc(P, P, P, P, P, P, 1, 8, N, 64, 0, ctypes.c_float(0.125), 1, P, P, P, None)
    assert st == FA_ERR_TOO_LARGE
