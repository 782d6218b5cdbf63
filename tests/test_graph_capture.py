"""HIP graph capture of the whole path: the C ABI enqueues only kernels on the caller's
stream (no allocation, no memset, no synchronisation), so a forward + both backward
designs + a dropout forward/backward can be captured once and replayed.  Every replay,
with eager work and synchronisations in between, must reproduce the eager results bit
for bit (the 5-GEMM dQ, summed with atomics, to within fp32 reordering)."""
import math

import pytest
import torch

from parity_util import make_inputs, note

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]


def test_fwd_bwd_replays_match_eager():
    from exact_attention_102_amd import (FA_BWD_5GEMM_ATOMIC, FA_BWD_7GEMM, fa_bwd, fa_bwd_dropout,
                                         fa_bwd_workspace_size, fa_fwd, fa_fwd_dropout)
    B, H, N, d = 2, 4, 384, 128
    scale = 1.0 / math.sqrt(d)
    dev, _, _ = make_inputs(B, H, N, d, seed=71)
    q, k, v, do = dev
    f32 = dict(dtype=torch.float32, device="cuda")
    o, o2 = (torch.empty((B, H, N, d), **f32) for _ in range(2))
    lse, lse2 = (torch.empty((B, H, N), **f32) for _ in range(2))
    g5, g7, gd = ([torch.empty((B, H, N, d), **f32) for _ in range(3)] for _ in range(3))
    ws = torch.empty(fa_bwd_workspace_size(B, H, N, d, FA_BWD_7GEMM), dtype=torch.uint8, device="cuda")

    def path(stream):
        fa_fwd(q, k, v, True, scale, o=o, lse=lse, stream=stream)
        fa_bwd(q, k, v, o, lse, do, True, scale, FA_BWD_5GEMM_ATOMIC, *g5, workspace=ws, stream=stream)
        fa_bwd(q, k, v, o, lse, do, True, scale, FA_BWD_7GEMM, *g7, workspace=ws, stream=stream)
        fa_fwd_dropout(q, k, v, False, scale, 0.2, 99, 1, o=o2, lse=lse2, stream=stream)
        fa_bwd_dropout(q, k, v, o2, lse2, do, False, scale, 0.2, 99, 1, FA_BWD_7GEMM, *gd, workspace=ws,
                       stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [t.clone() for t in [o, lse, o2, lse2, *g5, *g7, *gd]]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        note("replay %d" % rep)
        for t in [o, lse, o2, lse2, *g5, *g7, *gd]:
            t.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o, lse, o2, lse2, *g5, *g7, *gd]
        for i, (a, b) in enumerate(zip(got, eager)):
            if i == 4:                     # 5-GEMM dq: fp32 atomics, order varies
                assert torch.allclose(a, b, rtol=1e-5, atol=1e-6), "replay %d: 5-GEMM dq" % rep
            else:
                assert torch.equal(a, b), "replay %d: output %d differs" % (rep, i)
