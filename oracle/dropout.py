"""Attention with dropout on P, and the counter-based generator that draws its mask.

TEST INFRASTRUCTURE ONLY -- the same rules as ``oracle/attention.py``: only
``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import it; it shares no code with the HIP path.

What is computed, and where the pages say so
--------------------------------------------
* "ELI5: FlashAttention", standard-attention highlights: unfused attention spends
  its time in elementwise passes over the N x N matrix -- masking, softmax and
  dropout -- and FlashAttention fuses them into the kernel.  Dropout here is the
  usual inverted dropout on the attention probabilities: each P_ij is kept with
  probability 1 - p and scaled by the reciprocal of that probability, otherwise zeroed.
* The pages give no random-number specification.  Reading:
  the keep decision for score element (b, h, i, j) comes from the counter-based
  generator Philox4x32-10 of Salmon, Moraes, Dror and Shaw, "Parallel Random
  Numbers: As Easy as 1, 2, 3" (SC '11), so any kernel can recompute any
  element's decision from its coordinates without storing a mask.  One call
  yields 128 bits, read as eight 16-bit draws, one per key of an aligned group
  of eight keys:
      key     = (seed mod 2^32, seed div 2^32)
      counter = (j div 8, i, b * H + h, offset)
      draw    = 16-bit half (j mod 2) of word ((j mod 8) div 2), low half first
      t       = floor(p * 2^16), at most 2^16 - 1
      keep    = draw >= t
  so the drop probability is t / 2^16 (p rounded down to a multiple of 2^-16)
  and kept probabilities are scaled by s = 2^16 / (2^16 - t), the reciprocal of
  the exact keep probability, which keeps O unbiased.
* Forward: O = (P * M * s) V with M the keep mask; the log-sum-exp is that of
  the undropped scores (dropout acts after the softmax normalisation).
* Backward of L = sum(dO * O): with Pd = P * M * s,
      dV = Pd^T dO,  dPd = dO V^T,  dP = dPd * M * s,
      dS = P * (dP - rowsum(P * dP)),  dQ = scale dS K,  dK = scale dS^T Q.
  rowsum(P * dP) = rowsum(Pd * dPd) = rowsum(dO * O), so the kernels' row term
  (computed from O and dO) is unchanged by dropout; the tests check that identity.

Philox4x32-10 (from the paper's definition): ten rounds over four 32-bit words.
A round multiplies word 0 by 0xD2511F53 and word 2 by 0xCD9E8D57 (full 64-bit
products) and outputs (hi(w2 m1) ^ w1 ^ k0, lo(w2 m1), hi(w0 m0) ^ w3 ^ k1,
lo(w0 m0)); between rounds the key is bumped by the Weyl constants (0x9E3779B9,
0xBB67AE85) modulo 2^32.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, score_matrix, softmax_rows

__all__ = ["philox4x32_10", "keep_threshold", "keep_scale", "dropout_keep_mask", "attention_forward_dropout",
           "attention_backward_dropout", "attention_forward_dropout_batched", "attention_backward_dropout_batched"]

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32-10 on arrays of counters (broadcast); returns four uint32 arrays."""
    w = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = w[0] * _M0          # < 2^64: both factors < 2^32
        p1 = w[2] * _M1
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        w = [hi1 ^ w[1] ^ k0, lo1, hi0 ^ w[3] ^ k1, lo0]
    return [x.astype(np.uint32) for x in w]


def keep_threshold(p: float) -> int:
    """t = floor(p * 2^16), capped at 2^16 - 1, for p in [0, 1): an element is kept iff its draw >= t."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(np.floor(p * 65536.0)), 0xFFFF)


def keep_scale(p: float) -> float:
    """Factor on kept probabilities: 2^16 / (2^16 - t), the reciprocal of the keep probability."""
    return 65536.0 / (65536 - keep_threshold(p))


def dropout_keep_mask(bh: int, rows, n_keys: int, p: float, seed: int, offset: int = 0) -> np.ndarray:
    """Keep mask [len(rows), n_keys] (bool) of head index bh = b * H + h for query rows ``rows``."""
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(n_keys, dtype=np.int64)
    ci = np.broadcast_to(rows[:, None], (rows.size, n_keys))
    cj = np.broadcast_to(j[None, :] >> 3, (rows.size, n_keys))
    words = philox4x32_10(cj, ci, np.int64(bh), np.int64(offset), seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    word = np.choose(np.broadcast_to((j[None, :] & 7) >> 1, (rows.size, n_keys)), words)
    draw = (word >> np.broadcast_to(16 * (j[None, :] & 1), (rows.size, n_keys)).astype(np.uint32)) & np.uint32(0xFFFF)
    return draw >= np.uint32(keep_threshold(p))


def attention_forward_dropout(q, k, v, scale: float, causal: bool, p: float, seed: int, offset: int = 0, bh: int = 0,
                              row_chunk: int = 256):
    """One head (index bh): O = (P * M * s) V and the undropped natural-log LSE."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    n = q.shape[0]
    o = np.empty((n, v.shape[1]))
    lse = np.empty(n)
    inv_keep = keep_scale(p)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        prob, l = softmax_rows(score_matrix(q[r0:r1], k, scale, causal, r0))
        m = dropout_keep_mask(bh, np.arange(r0, r1), k.shape[0], p, seed, offset)
        o[r0:r1] = (prob * m * inv_keep) @ v
        lse[r0:r1] = l
    return o, lse


def attention_backward_dropout(q, k, v, do, scale: float, causal: bool, p: float, seed: int, offset: int = 0,
                               bh: int = 0, row_chunk: int = 256, return_rowterm: bool = False):
    """One head: gradients of L = sum(dO * O) for the dropout forward above (explicit chain rule)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rowterm = np.empty(n)
    inv_keep = keep_scale(p)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        prob, _ = softmax_rows(score_matrix(q[r0:r1], k, scale, causal, r0))
        mk = dropout_keep_mask(bh, np.arange(r0, r1), k.shape[0], p, seed, offset) * inv_keep
        pd = prob * mk
        dv += pd.T @ do[r0:r1]
        dpd = do[r0:r1] @ v.T
        dp = dpd * mk
        t = np.sum(prob * dp, axis=1, keepdims=True)
        ds = prob * (dp - t)
        dq[r0:r1] = float(scale) * (ds @ k)
        dk += float(scale) * (ds.T @ q[r0:r1])
        rowterm[r0:r1] = t[:, 0]
    if return_rowterm:
        return dq, dk, dv, rowterm
    return dq, dk, dv


def attention_forward_dropout_batched(q, k, v, scale, causal, p, seed, offset=0):
    """[B, H, N, d] -> (o, lse); head index b * H + h feeds the generator's counter."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    b, h, n, d = q.shape
    o = np.empty((b, h, n, v.shape[-1]))
    lse = np.empty((b, h, n))
    for i in range(b * h):
        o[i // h, i % h], lse[i // h, i % h] = attention_forward_dropout(q[i // h, i % h], k[i // h, i % h],
                                                                         v[i // h, i % h], scale, causal, p, seed,
                                                                         offset, bh=i)
    return o, lse


def attention_backward_dropout_batched(q, k, v, do, scale, causal, p, seed, offset=0):
    """[B, H, N, d] -> (dq, dk, dv) for the dropout forward."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    b, h = q.shape[:2]
    out = [np.empty(q.shape), np.empty(k.shape), np.empty(v.shape)]
    for i in range(b * h):
        g = attention_backward_dropout(q[i // h, i % h], k[i // h, i % h], v[i // h, i % h], do[i // h, i % h],
                                       scale, causal, p, seed, offset, bh=i)
        for t, x in zip(out, g):
            t[i // h, i % h] = x
    return tuple(out)
