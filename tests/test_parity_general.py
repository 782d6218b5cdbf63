"""GPU parity of the general entry points (any head dim 1..384, strided views)
against the fp64 oracle, at the same bar as the fixed-shape path: O max-abs
<= 1e-2, LSE max-abs <= 1e-3, dQ/dK/dV relative L2 <= 2e-2.

Head dims that are not built directly run on zero-padded copies at the next built
size; strided views cover a [B, N, H, d] layout seen as [B, H, N, d] and a packed
[B, N, 3, H, d] q/k/v tensor.
"""
import math

import pytest
import torch

from parity_util import VARIANTS, check_backward, check_forward, make_inputs, note, oracle_backward, oracle_forward

pytestmark = [pytest.mark.gpu, pytest.mark.usefixtures("require_gpu")]


def run_general(q, k, v, do, causal, scale, outs_bnhd=False):
    from exact_attention_102_amd import fa_bwd_general, fa_fwd_general
    B, H, N, d = q.shape
    o = lse = None
    if outs_bnhd:
        o = torch.empty((B, N, H, d), dtype=torch.float32, device=q.device).transpose(1, 2)
    o, lse = fa_fwd_general(q, k, v, causal, scale, o=o)
    torch.cuda.synchronize()
    grads = {}
    for name, var in VARIANTS.items():
        outs = [None, None, None]
        if outs_bnhd:
            outs = [torch.empty((B, N, H, d), dtype=torch.float32, device=q.device).transpose(1, 2) for _ in range(3)]
        grads[name] = fa_bwd_general(q, k, v, o, lse, do, causal, scale, var, dq=outs[0], dk=outs[1], dv=outs[2])
        torch.cuda.synchronize()
    return o, lse, grads


@pytest.mark.parametrize("d", [8, 40, 96, 127, 192, 250, 257, 300, 320, 383])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bhn", [(1, 2, 77), (2, 1, 300)], ids=lambda t: "B%dH%dN%d" % t)
def test_general_head_dims(d, causal, bhn):
    B, H, N = bhn
    scale = 1.0 / math.sqrt(d)
    note("general d=%d causal=%d B=%d H=%d N=%d" % (d, causal, B, H, N))
    dev, host, _ = make_inputs(B, H, N, d, seed=300 + d + N)
    o, lse, grads = run_general(*dev, causal, scale)
    check_forward(o.contiguous(), lse, *oracle_forward(host, scale, causal))
    refs = oracle_backward(host, scale, causal)
    for name, g in grads.items():
        note("  bwd %s" % name)
        check_backward([t.contiguous() for t in g], refs)


@pytest.mark.parametrize("d", [128, 96, 352])
@pytest.mark.parametrize("causal", [False, True])
def test_general_bnhd_views(d, causal):
    """Inputs and outputs stored [B, N, H, d] and passed as [B, H, N, d] views."""
    B, H, N = 2, 3, 200
    scale = 1.0 / math.sqrt(d)
    note("bnhd views d=%d causal=%d" % (d, causal))
    dev, host, _ = make_inputs(B, H, N, d, seed=41 + d)
    views = [x.transpose(1, 2).contiguous().transpose(1, 2) for x in dev]
    assert not views[0].is_contiguous()
    o, lse, grads = run_general(*views, causal, scale, outs_bnhd=True)
    check_forward(o.contiguous(), lse, *oracle_forward(host, scale, causal))
    refs = oracle_backward(host, scale, causal)
    for name, g in grads.items():
        note("  bwd %s" % name)
        check_backward([t.contiguous() for t in g], refs)


def test_general_packed_qkv():
    """q, k, v as slices of one packed [B, N, 3, H, d] tensor (row stride 3 H d)."""
    B, H, N, d = 1, 4, 160, 64
    scale = 1.0 / math.sqrt(d)
    note("packed qkv")
    dev, host, _ = make_inputs(B, H, N, d, seed=77)
    packed = torch.stack([x.transpose(1, 2) for x in dev[:3]], dim=2).contiguous()   # [B, N, 3, H, d]
    q, k, v = (packed[:, :, i].transpose(1, 2) for i in range(3))
    assert q.stride(2) == 3 * H * d
    for causal in (False, True):
        o, lse, grads = run_general(q, k, v, dev[3], causal, scale)
        check_forward(o.contiguous(), lse, *oracle_forward(host, scale, causal))
        refs = oracle_backward(host, scale, causal)
        for g in grads.values():
            check_backward([t.contiguous() for t in g], refs)


def test_general_native_contiguous_matches_fixed_entry():
    """With d = 128 and contiguous tensors the general entry takes the direct path: bit-identical
    results to fa_fwd / fa_bwd (7-GEMM, which is deterministic)."""
    from exact_attention_102_amd import FA_BWD_7GEMM, fa_bwd, fa_fwd
    B, H, N, d = 1, 2, 256, 128
    scale = 1.0 / math.sqrt(d)
    dev, _, _ = make_inputs(B, H, N, d, seed=5)
    o1, l1 = fa_fwd(*dev[:3], True, scale)
    o2, l2, grads = run_general(*dev, True, scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = fa_bwd(*dev[:3], o1, l1, dev[3], True, scale, FA_BWD_7GEMM)
    for a, b in zip(g1, grads["7gemm"]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,pitch", [(96, 128), (40, 64), (64, 72), (64, 68)])
@pytest.mark.parametrize("causal", [False, True])
def test_general_rows_wider_than_head_dim(d, pitch, causal):
    """Views of the first d columns of [B, H, N, pitch] buffers whose other columns hold NaN.
    Aligned pitches (128, 64, 72 elements) run in place, the kernels padding the head dim
    themselves; pitch 68 (136-byte rows) takes the padded-copy path.  Nothing past column d may be
    read (a NaN would spread into every result) or written (the NaNs must survive)."""
    from exact_attention_102_amd import fa_bwd_general, fa_fwd_general
    B, H, N = 2, 2, 130
    scale = 1.0 / math.sqrt(d)
    note("wide rows d=%d pitch=%d causal=%d" % (d, pitch, causal))
    dev, host, _ = make_inputs(B, H, N, d, seed=900 + d + pitch)

    def wide(x, dtype):
        buf = torch.full((B, H, N, pitch), float("nan"), dtype=dtype, device="cuda")
        if x is not None:
            buf[..., :d] = x
        return buf

    bufs = [wide(x, torch.bfloat16) for x in dev]
    views = [b[..., :d] for b in bufs]
    obuf = wide(None, torch.float32)
    o, lse = fa_fwd_general(*views[:3], causal, scale, o=obuf[..., :d])
    torch.cuda.synchronize()
    assert torch.isnan(obuf[..., d:]).all()
    check_forward(o.contiguous(), lse, *oracle_forward(host, scale, causal))
    refs = oracle_backward(host, scale, causal)
    for name, var in VARIANTS.items():
        note("  bwd %s" % name)
        gbufs = [wide(None, torch.float32) for _ in range(3)]
        if var == VARIANTS["5gemm"]:
            for gb in gbufs:               # the atomic dq accumulates into what the library clears
                gb[..., :d] = 123.0
        g = fa_bwd_general(*views[:3], o, lse, views[3], causal, scale, var, dq=gbufs[0][..., :d],
                           dk=gbufs[1][..., :d], dv=gbufs[2][..., :d])
        torch.cuda.synchronize()
        for gb in gbufs:
            assert torch.isnan(gb[..., d:]).all()
        check_backward([t.contiguous() for t in g], refs)
