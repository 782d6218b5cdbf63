"""Thin ctypes binding over libfa.so (include/fa.h): argument marshalling only.

Every step of the attention computation runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and the stream; nothing here computes.
If libfa.so is missing the binding raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4
FA_ERR_TOO_LARGE = 5
FA_NOALLOC_MAX_ROWS = 1 << 23
FA_BWD_5GEMM_ATOMIC = 0
FA_BWD_7GEMM = 1
PASS_FWD, PASS_DKDV, PASS_DKDV_ATOMIC, PASS_DQ = 0, 1, 2, 3

_lib = None


class FaStrides(ctypes.Structure):
    """fa_strides: element strides (b, h, n) of a [B, H, N, d] view with a contiguous head dim."""
    _fields_ = [("b", ctypes.c_longlong), ("h", ctypes.c_longlong), ("n", ctypes.c_longlong)]


class FaDropout(ctypes.Structure):
    """fa_dropout: drop probability p in [0, 1), 64-bit generator seed, 32-bit counter offset."""
    _fields_ = [("p", ctypes.c_double), ("seed", ctypes.c_ulonglong), ("offset", ctypes.c_uint)]


class FAError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s" % (what, fa_status_string(status)))
        self.status = status


def lib() -> ctypes.CDLL:
    """Loads libfa.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libfa.so is not built (%s); run __graft_entry__.build() or "
                           "python -m exact_attention_102_amd.build" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz, cp = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_char_p
    L.fa_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, f, vp, vp, vp]
    L.fa_fwd.restype = i
    L.fa_fwd_ex.argtypes = [vp, vp, vp, i, i, i, i, i, f, vp, vp, vp, i]
    L.fa_fwd_ex.restype = i
    L.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_bwd_workspace_size.restype = sz
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, vp, sz, vp]
    L.fa_bwd.restype = i
    L.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, vp, sz, vp, i, i]
    L.fa_bwd_ex.restype = i
    L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, vp]
    L.fa_bwd_noalloc.restype = i
    L.fa_bwd_preprocess.argtypes = [vp, vp, i, i, i, i, vp, vp, i, vp]
    L.fa_bwd_preprocess.restype = i
    L.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, vp, vp, vp, i]
    L.fa_bwd_dkdv.restype = i
    L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, i]
    L.fa_bwd_dq.restype = i
    L.fa_bwd_dq_delta.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, vp, i]
    L.fa_bwd_dq_delta.restype = i
    L.fa_num_configs.argtypes = [i, i, i]
    L.fa_num_configs.restype = i
    L.fa_config_name.argtypes = [i, i, i, i, cp, sz]
    L.fa_config_name.restype = i
    L.fa_default_config.argtypes = [i, i, i]
    L.fa_default_config.restype = i
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = cp
    L.fa_version.argtypes = []
    L.fa_version.restype = cp
    st = FaStrides
    L.fa_fwd_general_workspace_size.argtypes = [i, i, i, i]
    L.fa_fwd_general_workspace_size.restype = sz
    L.fa_bwd_general_workspace_size.argtypes = [i, i, i, i, i]
    L.fa_bwd_general_workspace_size.restype = sz
    L.fa_fwd_general.argtypes = [vp, st, vp, st, vp, st, i, i, i, i, i, f, vp, st, vp, vp, sz, vp]
    L.fa_fwd_general.restype = i
    L.fa_bwd_general.argtypes = [vp, st, vp, st, vp, st, vp, st, vp, vp, st, i, i, i, i, i, f, i,
                                 vp, st, vp, st, vp, st, vp, sz, vp]
    L.fa_bwd_general.restype = i
    dr = FaDropout
    L.fa_fwd_dropout.argtypes = [vp, vp, vp, i, i, i, i, i, f, dr, vp, vp, vp]
    L.fa_fwd_dropout.restype = i
    L.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, dr, i, vp, vp, vp, vp, sz, vp]
    L.fa_bwd_dropout.restype = i
    L.fa_dropout_keep_scale.argtypes = [ctypes.c_double]
    L.fa_dropout_keep_scale.restype = ctypes.c_double
    L.fa_fwd_general_dropout.argtypes = [vp, st, vp, st, vp, st, i, i, i, i, i, f, dr, vp, st, vp, vp, sz, vp]
    L.fa_fwd_general_dropout.restype = i
    L.fa_bwd_general_dropout.argtypes = [vp, st, vp, st, vp, st, vp, st, vp, vp, st, i, i, i, i, i, f, dr, i,
                                         vp, st, vp, st, vp, st, vp, sz, vp]
    L.fa_bwd_general_dropout.restype = i
    _lib = L
    return L


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def fa_version() -> str:
    return lib().fa_version().decode()


def fa_num_configs(pass_id: int, d: int, causal: bool = False) -> int:
    return lib().fa_num_configs(int(pass_id), int(d), int(bool(causal)))


def fa_config_name(pass_id: int, d: int, causal: bool, index: int) -> str:
    buf = ctypes.create_string_buffer(128)
    if lib().fa_config_name(int(pass_id), int(d), int(bool(causal)), int(index), buf, 128) != 0:
        raise IndexError("no configuration %d for pass %d, d=%d" % (index, pass_id, d))
    return buf.value.decode()


def fa_default_config(pass_id: int, d: int, causal: bool = False) -> int:
    return lib().fa_default_config(int(pass_id), int(d), int(bool(causal)))


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int, variant: int = FA_BWD_7GEMM) -> int:
    return int(lib().fa_bwd_workspace_size(int(B), int(H), int(N), int(d), int(variant)))


# --------------------------------------------------------------------------- torch marshalling
def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _check(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (cuda/HIP) tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous [B, H, N, d]" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return ctypes.c_void_p(t.data_ptr())


def _fwd_args(q, k, v, o, lse):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    pq = _check(q, "q", torch.bfloat16)
    pk = _check(k, "k", torch.bfloat16, q.shape)
    pv = _check(v, "v", torch.bfloat16, q.shape)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    po = _check(o, "o", torch.float32, q.shape)
    pl = _check(lse, "lse", torch.float32, (B, H, N))
    return (B, H, N, d), (pq, pk, pv), (po, pl), (o, lse)


def fa_fwd(q, k, v, causal: bool, scale: float, o=None, lse=None, stream=None, cfg: int = -1):
    """Forward: returns (o fp32 [B,H,N,d], lse fp32 [B,H,N]); allocates outputs if not given."""
    dims, ins, outs, res = _fwd_args(q, k, v, o, lse)
    st = lib().fa_fwd_ex(*ins, *dims, int(bool(causal)), float(scale), *outs, _stream_ptr(stream), int(cfg))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return res


def fa_fwd_dropout(q, k, v, causal: bool, scale: float, p: float, seed: int, offset: int = 0, o=None, lse=None,
                   stream=None):
    """Forward with dropout on P (include/fa.h, fa_fwd_dropout): returns (o, lse)."""
    dims, ins, outs, res = _fwd_args(q, k, v, o, lse)
    drop = FaDropout(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF)
    st = lib().fa_fwd_dropout(*ins, *dims, int(bool(causal)), float(scale), drop, *outs, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_dropout")
    return res


def fa_dropout_keep_scale(p: float) -> float:
    """Factor on kept probabilities for drop probability p (65536 / (65536 - floor(p 65536)))."""
    r = lib().fa_dropout_keep_scale(float(p))
    if r < 0:
        raise ValueError("dropout probability must be in [0, 1)")
    return r


def _bwd_args(q, k, v, o, lse, dout, variant, dq, dk, dv, workspace):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    ptr = [_check(q, "q", torch.bfloat16), _check(k, "k", torch.bfloat16, q.shape),
           _check(v, "v", torch.bfloat16, q.shape), _check(o, "o", torch.float32, q.shape),
           _check(lse, "lse", torch.float32, (B, H, N)), _check(dout, "dout", torch.bfloat16, q.shape)]
    outs = []
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        if t is None:
            t = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
        outs.append(t)
    pouts = [_check(t, n, torch.float32, q.shape) for t, n in zip(outs, ("dq", "dk", "dv"))]
    need = fa_bwd_workspace_size(B, H, N, d, variant)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    return (B, H, N, d), ptr, pouts, (ctypes.c_void_p(workspace.data_ptr()), ws_bytes), tuple(outs)


def fa_bwd(q, k, v, o, lse, dout, causal: bool, scale: float, variant: int = FA_BWD_7GEMM,
           dq=None, dk=None, dv=None, workspace=None, stream=None, cfg_dkdv: int = -1, cfg_dq: int = -1):
    """Backward: returns (dq, dk, dv), fp32 [B,H,N,d]; allocates outputs/workspace if not given."""
    dims, ptr, pouts, ws, res = _bwd_args(q, k, v, o, lse, dout, variant, dq, dk, dv, workspace)
    st = lib().fa_bwd_ex(*ptr, *dims, int(bool(causal)), float(scale), int(variant), *pouts, *ws,
                         _stream_ptr(stream), int(cfg_dkdv), int(cfg_dq))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return res


def fa_bwd_noalloc(q, k, v, o, lse, dout, causal: bool, scale: float, variant: int, dq, dk, dv, stream=None):
    """fa_bwd_noalloc: the backward with the library's fixed scratch instead of a workspace; the caller
    provides every output (nothing is allocated here either).  Returns (dq, dk, dv)."""
    torch = _torch()
    if dq is None or dk is None or dv is None:
        raise ValueError("fa_bwd_noalloc writes into caller-provided dq, dk, dv")
    B, H, N, d = q.shape
    ptr = [_check(q, "q", torch.bfloat16), _check(k, "k", torch.bfloat16, q.shape),
           _check(v, "v", torch.bfloat16, q.shape), _check(o, "o", torch.float32, q.shape),
           _check(lse, "lse", torch.float32, (B, H, N)), _check(dout, "dout", torch.bfloat16, q.shape)]
    pouts = [_check(t, n, torch.float32, q.shape) for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"))]
    st = lib().fa_bwd_noalloc(*ptr, B, H, N, d, int(bool(causal)), float(scale), int(variant), *pouts,
                              _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_noalloc")
    return dq, dk, dv


def fa_bwd_dropout(q, k, v, o, lse, dout, causal: bool, scale: float, p: float, seed: int, offset: int = 0,
                   variant: int = FA_BWD_7GEMM, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward of the dropout forward (same p, seed, offset): returns (dq, dk, dv)."""
    dims, ptr, pouts, ws, res = _bwd_args(q, k, v, o, lse, dout, variant, dq, dk, dv, workspace)
    drop = FaDropout(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF)
    st = lib().fa_bwd_dropout(*ptr, *dims, int(bool(causal)), float(scale), drop, int(variant), *pouts, *ws,
                              _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dropout")
    return res


def fa_bwd_preprocess(o, dout, delta=None, dq=None, stream=None):
    """delta[b,h,i] = sum_k dout * o (and zeroes dq when given); returns delta."""
    torch = _torch()
    B, H, N, d = o.shape
    po = _check(o, "o", torch.float32)
    pd = _check(dout, "dout", torch.bfloat16, o.shape)
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=o.device)
    pdel = _check(delta, "delta", torch.float32, (B, H, N))
    pdq = _check(dq, "dq", torch.float32, o.shape) if dq is not None else ctypes.c_void_p(0)
    st = lib().fa_bwd_preprocess(po, pd, B, H, N, d, pdel, pdq, int(dq is not None), _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_preprocess")
    return delta


def fa_bwd_dkdv(q, k, v, dout, lse, delta, causal: bool, scale: float, atomic_dq: bool, dk, dv, dq=None,
                stream=None, cfg: int = -1):
    """dK/dV kernel stage (plus fp32-atomic dQ when atomic_dq); outputs must be allocated by the caller."""
    torch = _torch()
    B, H, N, d = q.shape
    ptr = [_check(q, "q", torch.bfloat16), _check(k, "k", torch.bfloat16, q.shape),
           _check(v, "v", torch.bfloat16, q.shape), _check(dout, "dout", torch.bfloat16, q.shape),
           _check(lse, "lse", torch.float32, (B, H, N)), _check(delta, "delta", torch.float32, (B, H, N))]
    pq = _check(dq, "dq", torch.float32, q.shape) if atomic_dq else ctypes.c_void_p(0)
    st = lib().fa_bwd_dkdv(*ptr, B, H, N, d, int(bool(causal)), float(scale), int(bool(atomic_dq)), pq,
                           _check(dk, "dk", torch.float32, q.shape), _check(dv, "dv", torch.float32, q.shape),
                           _stream_ptr(stream), int(cfg))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dkdv")
    return dk, dv


def fa_bwd_dq(q, k, v, dout, lse, delta, causal: bool, scale: float, dq, stream=None, cfg: int = -1):
    """dQ kernel stage of the 7-GEMM design; dq must be allocated by the caller."""
    torch = _torch()
    B, H, N, d = q.shape
    ptr = [_check(q, "q", torch.bfloat16), _check(k, "k", torch.bfloat16, q.shape),
           _check(v, "v", torch.bfloat16, q.shape), _check(dout, "dout", torch.bfloat16, q.shape),
           _check(lse, "lse", torch.float32, (B, H, N)), _check(delta, "delta", torch.float32, (B, H, N))]
    st = lib().fa_bwd_dq(*ptr, B, H, N, d, int(bool(causal)), float(scale), _check(dq, "dq", torch.float32, q.shape),
                         _stream_ptr(stream), int(cfg))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dq")
    return dq


def fa_bwd_dq_delta(q, k, v, o, dout, lse, causal: bool, scale: float, delta, dq, stream=None, cfg: int = -1):
    """7-GEMM dQ kernel that computes delta itself from o and dout and writes it (for
    fa_bwd_dkdv, run after it); delta and dq must be allocated by the caller."""
    torch = _torch()
    B, H, N, d = q.shape
    ptr = [_check(q, "q", torch.bfloat16), _check(k, "k", torch.bfloat16, q.shape),
           _check(v, "v", torch.bfloat16, q.shape), _check(o, "o", torch.float32, q.shape),
           _check(dout, "dout", torch.bfloat16, q.shape), _check(lse, "lse", torch.float32, (B, H, N))]
    st = lib().fa_bwd_dq_delta(*ptr, B, H, N, d, int(bool(causal)), float(scale),
                               _check(delta, "delta", torch.float32, (B, H, N)),
                               _check(dq, "dq", torch.float32, q.shape), _stream_ptr(stream), int(cfg))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dq_delta")
    return delta, dq


# --------------------------------------------------------------------------- general entry points
def _view(t, name, dtype, shape):
    """Pointer and strides of a [B, H, N, d] view whose last dimension is contiguous."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a device torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.stride(3) != 1 and t.shape[3] > 1:
        raise ValueError("%s: the head dimension must be contiguous (stride 1)" % name)
    return ctypes.c_void_p(t.data_ptr()), FaStrides(t.stride(0), t.stride(1), t.stride(2))


def fa_fwd_general_workspace_size(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_fwd_general_workspace_size(int(B), int(H), int(N), int(d)))


def fa_bwd_general_workspace_size(B: int, H: int, N: int, d: int, variant: int = FA_BWD_7GEMM) -> int:
    return int(lib().fa_bwd_general_workspace_size(int(B), int(H), int(N), int(d), int(variant)))


def _workspace(need, device, workspace):
    torch = _torch()
    if workspace is None:
        workspace = torch.empty(max(int(need), 16), dtype=torch.uint8, device=device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return workspace, ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size()


def _dropout_arg(dropout):
    """(p, seed[, offset]) or FaDropout -> FaDropout."""
    if isinstance(dropout, FaDropout):
        return dropout
    p, seed = dropout[0], dropout[1]
    off = dropout[2] if len(dropout) > 2 else 0
    return FaDropout(float(p), int(seed) & 0xFFFFFFFFFFFFFFFF, int(off) & 0xFFFFFFFF)


def fa_fwd_general(q, k, v, causal: bool, scale: float, o=None, lse=None, workspace=None, stream=None,
                   dropout=None):
    """Forward for any head dim 1..384 and strided [B, H, N, d] views (e.g. a [B, N, H, d] tensor
    transposed); returns (o, lse).  o defaults to a new contiguous fp32 tensor.  dropout = (p, seed,
    offset) runs fa_fwd_general_dropout."""
    torch = _torch()
    B, H, N, d = q.shape
    pq, sq = _view(q, "q", torch.bfloat16, q.shape)
    pk, sk = _view(k, "k", torch.bfloat16, q.shape)
    pv, sv = _view(v, "v", torch.bfloat16, q.shape)
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    po, so = _view(o, "o", torch.float32, q.shape)
    pl = _check(lse, "lse", torch.float32, (B, H, N))
    workspace, pw, wb = _workspace(fa_fwd_general_workspace_size(B, H, N, d), q.device, workspace)
    if dropout is None:
        st = lib().fa_fwd_general(pq, sq, pk, sk, pv, sv, B, H, N, d, int(bool(causal)), float(scale), po, so, pl, pw,
                                  wb, _stream_ptr(stream))
    else:
        st = lib().fa_fwd_general_dropout(pq, sq, pk, sk, pv, sv, B, H, N, d, int(bool(causal)), float(scale),
                                          _dropout_arg(dropout), po, so, pl, pw, wb, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_general")
    return o, lse


def fa_bwd_general(q, k, v, o, lse, dout, causal: bool, scale: float, variant: int = FA_BWD_7GEMM,
                   dq=None, dk=None, dv=None, workspace=None, stream=None, dropout=None):
    """Backward for any head dim 1..384 and strided views; returns (dq, dk, dv) (new contiguous fp32
    tensors unless given).  dropout = the forward's (p, seed, offset) runs fa_bwd_general_dropout."""
    torch = _torch()
    B, H, N, d = q.shape
    args = [_view(q, "q", torch.bfloat16, q.shape), _view(k, "k", torch.bfloat16, q.shape),
            _view(v, "v", torch.bfloat16, q.shape), _view(o, "o", torch.float32, q.shape)]
    pl = _check(lse, "lse", torch.float32, (B, H, N))
    pdo, sdo = _view(dout, "dout", torch.bfloat16, q.shape)
    outs = [t if t is not None else torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
            for t in (dq, dk, dv)]
    pouts = [_view(t, n, torch.float32, q.shape) for t, n in zip(outs, ("dq", "dk", "dv"))]
    workspace, pw, wb = _workspace(fa_bwd_general_workspace_size(B, H, N, d, variant), q.device, workspace)
    flat = [x for pair in args for x in pair]
    flat_outs = [x for pair in pouts for x in pair]
    if dropout is None:
        st = lib().fa_bwd_general(*flat, pl, pdo, sdo, B, H, N, d, int(bool(causal)), float(scale), int(variant),
                                  *flat_outs, pw, wb, _stream_ptr(stream))
    else:
        st = lib().fa_bwd_general_dropout(*flat, pl, pdo, sdo, B, H, N, d, int(bool(causal)), float(scale),
                                          _dropout_arg(dropout), int(variant), *flat_outs, pw, wb, _stream_ptr(stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_general")
    return tuple(outs)
