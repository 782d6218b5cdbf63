"""GPU regression tests of fixed bugs, through the C ABI.

Atomic dQ rows past the end: the 5-GEMM kernels add dQ with fp32 buffer atomics and
rely on the buffer range check to drop the adds of query rows past N.  The check
covers the vector and immediate offsets only, so a row step carried in the scalar
offset escaped it: rows past the end then received (+0.0) adds in the next head's
accumulator or past the end of dq.  Here dq sits at the front of a larger buffer whose
tail holds -0.0; an add of +0.0 turns -0.0 into +0.0, so any stray add flips a sign
bit without changing a value's magnitude (and nothing faults: the tail is allocated).
"""
import math

import numpy as np
import pytest
import torch

from parity_util import (VARIANTS, check_backward, gpu_forward, make_inputs, note, oracle_backward)

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]

NEG_ZERO_BITS = -0x80000000  # int32 view of -0.0


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("N", [33, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_atomic_dq_adds_stay_inside_dq(d, N, causal):
    from exact_attention_102_amd import PASS_DKDV_ATOMIC, fa_bwd, fa_config_name, fa_num_configs
    B, H = 1, 2
    scale = 1.0 / math.sqrt(d)
    dev, host, _ = make_inputs(B, H, N, d, seed=41 + N + d)
    o, lse = gpu_forward(dev, causal, scale)
    refs = oracle_backward(host, scale, causal)
    elems = B * H * N * d
    tail = 64 * 256
    buf = torch.empty(elems + tail, dtype=torch.float32, device="cuda")
    dq = buf[:elems].view(B, H, N, d)
    dk = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    for c in range(fa_num_configs(PASS_DKDV_ATOMIC, d)):
        note("atomic dq bounds d=%d N=%d causal=%d cfg %d (%s)" % (d, N, causal, c,
                                                                  fa_config_name(PASS_DKDV_ATOMIC, d, causal, c)))
        buf.fill_(-0.0)
        q, k, v, do = dev
        fa_bwd(q, k, v, o, lse, do, causal, scale, VARIANTS["5gemm"], dq=dq, dk=dk, dv=dv, cfg_dkdv=c)
        torch.cuda.synchronize()
        bits = buf[elems:].view(torch.int32).cpu().numpy()
        stray = int(np.count_nonzero(bits != NEG_ZERO_BITS))
        assert stray == 0, "%d elements past the end of dq were written" % stray
        check_backward((dq, dk, dv), refs)
