"""Plain fp64 CPU oracle for exact scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The HIP product path
(``exact_attention_102_amd``) never imports, links or calls it, and this module
imports nothing from that package: the two share no code.

What is computed, and where the pages say so
--------------------------------------------
* "ELI5: FlashAttention" (A. Gordic), highlights on the standard implementation:
  attention is the score matrix S = Q K^T, a row softmax of S (with masking), and
  the product with V.  FlashAttention is *exact*: it reaches precisely the same
  result as that plain computation, only with fewer HBM round trips.  So this
  oracle IS the plain definition, materialising S and P in fp64.
* Same page, tiling highlights: a softmax split into key blocks is recovered
  exactly by carrying two statistics per block, m(x) (the maximum score) and
  l(x) (the sum of exponentials), and merging them with normalising
  coefficients.  ``online_softmax_stats`` and ``blockwise_attention_forward``
  follow that description step by step; tests pin them to the plain softmax.
* "Potential algorithmic improvements for backward pass" (flash-attention
  GitHub issue 1172), opening comment: the operands of the fused attention are
  Q, K, V, O, the log-sum-exp, dO, dV, dK and dQ.  The log-sum-exp is the one
  statistic the forward saves for the backward (``lse`` below).
* Same page, recomputation (and "ELI5", recomputation highlight): the backward
  recomputes S and P from Q, K.  Here the backward simply recomputes the plain
  softmax from Q, K and applies the chain rule for L = sum(dO * O):
      dV = P^T dO,  dP = dO V^T,  dS_i = (diag(P_i) - P_i P_i^T) dP_i,
      dQ = scale * dS K,  dK = scale * dS^T Q.

Readings where the pages are silent
-----------------------------------
* scale multiplies Q K^T before the softmax; causal means query i sees keys
  j <= i (N_q == N_k, so top-left and bottom-right alignment coincide); masked
  scores are -inf and contribute exactly 0.
* The log-sum-exp is the natural log: lse_i = log(sum_j exp(S_ij)).
* The softmax backward uses the literal Jacobian on tiny inputs
  (``attention_backward_jacobian``) and its identical closed form
  dS = P * (dP - rowsum(P * dP)) at scale.  The row term is computed here as
  rowsum(P * dP); the kernel's identity rowsum(P * dP) == rowsum(dO * O) is
  *checked* by the tests, never used by the oracle.
* Rows of S are independent, so the oracle evaluates query rows in chunks to
  bound memory (an N x N fp64 matrix is 2 GiB at N = 16384).  Chunking is not a
  blocking of the method: each row is the full definition.  dK and dV sum the
  chunk contributions, which only reorders fp64 additions.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "score_matrix",
    "softmax_rows",
    "attention_forward",
    "attention_backward",
    "attention_backward_jacobian",
    "attention_backward_key_rows",
    "attention_forward_batched",
    "attention_backward_batched",
    "online_softmax_stats",
    "blockwise_attention_forward",
    "usable_cores",
]


def usable_cores() -> int:
    """Number of host cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def score_matrix(q, k, scale: float, causal: bool, row_start: int = 0) -> np.ndarray:
    """S = scale * q k^T for query rows ``row_start .. row_start+len(q)-1`` of one head.

    Causal (reading: query i sees keys j <= i) sets S_ij = -inf for j > i.
    "ELI5: FlashAttention", standard-attention highlights: the score matrix and
    the masking step.
    """
    q = _f64(q)
    k = _f64(k)
    s = (q @ k.T) * float(scale)
    if causal:
        rows = np.arange(row_start, row_start + q.shape[0])[:, None]
        cols = np.arange(k.shape[0])[None, :]
        s = np.where(cols > rows, -np.inf, s)
    return s


def softmax_rows(s: np.ndarray):
    """Row softmax with max subtraction; returns (P, lse) with lse natural-log.

    P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i), m_i = max_j S_ij,
    lse_i = m_i + log(sum_j exp(S_ij - m_i)).  Every row has at least one finite
    entry (the diagonal under causal masking), so m_i is finite.
    """
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=1, keepdims=True)
    p = e / z
    lse = (m + np.log(z))[:, 0]
    return p, lse


def attention_forward(q, k, v, scale: float, causal: bool, row_chunk: int = 512):
    """One head: O = softmax(scale * Q K^T [masked]) V and the natural-log LSE.

    q, k, v: [N, d].  Returns (o [N, d], lse [N]) in fp64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n = q.shape[0]
    o = np.empty((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        p, l = softmax_rows(score_matrix(q[r0:r1], k, scale, causal, r0))
        o[r0:r1] = p @ v
        lse[r0:r1] = l
    return o, lse


def attention_backward(q, k, v, do, scale: float, causal: bool, row_chunk: int = 512,
                       return_rowterm: bool = False):
    """One head: gradients of L = sum(dO * O) with respect to Q, K, V.

    Recomputes P from Q and K (no saved statistics are trusted), then
        dV = P^T dO,  dP = dO V^T,
        dS = P * (dP - rowsum(P * dP))      (closed form of (diag P_i - P_i P_i^T) dP_i),
        dQ = scale * dS K,  dK = scale * dS^T Q.
    Masked entries have P = 0 and contribute nothing.  With ``return_rowterm``
    also returns rowsum(P * dP) per query row.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    n = q.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rowterm = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, row_chunk):
        r1 = min(n, r0 + row_chunk)
        p, _ = softmax_rows(score_matrix(q[r0:r1], k, scale, causal, r0))
        dv += p.T @ do[r0:r1]
        dp = do[r0:r1] @ v.T
        t = np.sum(p * dp, axis=1, keepdims=True)
        ds = p * (dp - t)
        dq[r0:r1] = float(scale) * (ds @ k)
        dk += float(scale) * (ds.T @ q[r0:r1])
        rowterm[r0:r1] = t[:, 0]
    if return_rowterm:
        return dq, dk, dv, rowterm
    return dq, dk, dv


def attention_backward_jacobian(q, k, v, do, scale: float, causal: bool):
    """Tiny-input backward with the literal softmax Jacobian per row.

    For each query row i: J_i = diag(P_i) - P_i P_i^T and dS_i = J_i dP_i.  Meant
    for N <= 128; it builds an N x N Jacobian per row.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    p, _ = softmax_rows(score_matrix(q, k, scale, causal, 0))
    dv = p.T @ do
    dp = do @ v.T
    ds = np.empty_like(p)
    for i in range(p.shape[0]):
        jac = np.diag(p[i]) - np.outer(p[i], p[i])
        ds[i] = jac @ dp[i]
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward_key_rows(q, k, v, do, scale: float, causal: bool, keys, row_chunk: int = 128,
                                workers: int | None = None):
    """One head: dK and dV of the key rows ``keys`` only, by the chain rule of ``attention_backward``.

    dV_j = sum_i P_ij dO_i and dK_j = scale * sum_i dS_ij q_i run over every query row i
    that attends to key j; each such row's P_i is its own full max-subtracted softmax (all
    its keys) and dS_i = P_i * (dP_i - rowsum(P_i * dP_i)) with dP_i = dO_i V^T, as in
    ``attention_backward``.  Under the causal mask (query i sees keys j <= i) only rows
    i >= min(keys) attend to a sampled key, so keys near the end of a long sequence need
    few rows; without the mask every row does.  Query rows are processed in chunks on a
    thread pool (rows are independent; the per-chunk sums only reorder fp64 additions).
    Returns (dk [len(keys), d], dv [len(keys), d]) in fp64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    keys = np.asarray(keys, dtype=np.int64)
    n = q.shape[0]
    first = int(keys.min()) if causal else 0
    starts = list(range(first, n, row_chunk))

    def part(r0):
        r1 = min(n, r0 + row_chunk)
        p, _ = softmax_rows(score_matrix(q[r0:r1], k, scale, causal, r0))
        dp = do[r0:r1] @ v.T
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        return p[:, keys].T @ do[r0:r1], float(scale) * (ds[:, keys].T @ q[r0:r1])

    workers = max(1, min(workers or usable_cores(), 8, len(starts)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        parts = list(ex.map(part, starts))
    dv = np.sum([a for a, _ in parts], axis=0)
    dk = np.sum([b for _, b in parts], axis=0)
    return dk, dv


def _map_heads(fn, n_heads: int, workers: int | None):
    workers = max(1, min(workers or usable_cores(), n_heads))
    if workers == 1:
        return [fn(i) for i in range(n_heads)]
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, range(n_heads)))


def attention_forward_batched(q, k, v, scale: float, causal: bool, workers: int | None = None,
                              heads=None, row_chunk: int = 512):
    """[B, H, N, d] inputs -> (o [B, H, N, d], lse [B, H, N]) in fp64.

    Heads are independent; a thread pool runs them in parallel (numpy releases
    the GIL inside BLAS and ufuncs).  ``heads`` optionally restricts the work to
    a list of flattened (b * H + h) indices; other heads are left as NaN.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    b, h, n, d = q.shape
    qf = q.reshape(b * h, n, d)
    kf = k.reshape(b * h, n, d)
    vf = v.reshape(b * h, n, v.shape[-1])
    o = np.full((b * h, n, v.shape[-1]), np.nan)
    lse = np.full((b * h, n), np.nan)
    idx = list(range(b * h)) if heads is None else list(heads)

    def one(t):
        i = idx[t]
        o[i], lse[i] = attention_forward(qf[i], kf[i], vf[i], scale, causal, row_chunk)

    _map_heads(one, len(idx), workers)
    return o.reshape(b, h, n, -1), lse.reshape(b, h, n)


def attention_backward_batched(q, k, v, do, scale: float, causal: bool, workers: int | None = None,
                               heads=None, row_chunk: int = 512):
    """[B, H, N, d] inputs -> (dq, dk, dv), each [B, H, N, d] fp64 (NaN outside ``heads``)."""
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    b, h, n, d = q.shape
    qf, kf, vf, dof = (x.reshape(b * h, n, x.shape[-1]) for x in (q, k, v, do))
    dq = np.full(qf.shape, np.nan)
    dk = np.full(kf.shape, np.nan)
    dv = np.full(vf.shape, np.nan)
    idx = list(range(b * h)) if heads is None else list(heads)

    def one(t):
        i = idx[t]
        dq[i], dk[i], dv[i] = attention_backward(qf[i], kf[i], vf[i], dof[i], scale, causal, row_chunk)

    _map_heads(one, len(idx), workers)
    return dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(v.shape)


def online_softmax_stats(block_scores):
    """Merge per-block softmax statistics of one score row, in the order given.

    "ELI5: FlashAttention", tiling highlights: each block x carries m(x), its
    maximum score, and l(x), the sum of exp(score - m(x)) over the block.  Two
    partial results (m1, l1), (m2, l2) combine as
        m = max(m1, m2),   l = exp(m1 - m) * l1 + exp(m2 - m) * l2.
    Returns (m, l) for the whole row; log(l) + m is its log-sum-exp.
    Blocks whose scores are all -inf (fully masked) carry l = 0 and are skipped.
    """
    m_run = -math.inf
    l_run = 0.0
    for blk in block_scores:
        blk = _f64(blk)
        if blk.size == 0:
            continue
        m_blk = float(np.max(blk))
        if m_blk == -math.inf:
            continue
        l_blk = float(np.sum(np.exp(blk - m_blk)))
        m_new = max(m_run, m_blk)
        l_run = math.exp(m_run - m_new) * l_run + math.exp(m_blk - m_new) * l_blk
        m_run = m_new
    return m_run, l_run


def blockwise_attention_forward(q, k, v, scale: float, causal: bool, block_sizes):
    """One head, forward computed key block by key block with the m/l merge.

    ``block_sizes`` partitions the N keys (any sizes, in order).  For each key
    block: block scores, block max and exp-sum, an unnormalised block output
    exp(S - m_blk) V_blk; the running (m, l, O) is merged with the block's by
    the normalising coefficients exp(m_old - m_new) and exp(m_blk - m_new), as
    the tiling highlights of "ELI5: FlashAttention" describe.  O is divided by
    l once at the end.  Returns (o, lse) like ``attention_forward``.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    n = q.shape[0]
    assert sum(block_sizes) == k.shape[0], "block sizes must partition the keys"
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, v.shape[1]))
    j0 = 0
    for bs in block_sizes:
        j1 = j0 + bs
        s = score_matrix(q, k[j0:j1], scale, False)
        if causal:
            rows = np.arange(n)[:, None]
            cols = np.arange(j0, j1)[None, :]
            s = np.where(cols > rows, -np.inf, s)
        m_blk = np.max(s, axis=1)
        live = m_blk > -np.inf
        m_safe = np.where(live, m_blk, 0.0)
        e = np.exp(s - m_safe[:, None])                   # zero on masked entries
        l_blk = np.sum(e, axis=1)
        o_blk = e @ v[j0:j1]
        m_new = np.maximum(m, m_blk)
        m_new_safe = np.where(np.isfinite(m_new), m_new, 0.0)
        a_old = np.where(np.isfinite(m), np.exp(m - m_new_safe), 0.0)
        a_blk = np.where(live, np.exp(m_blk - m_new_safe), 0.0)
        l = a_old * l + a_blk * l_blk
        o = a_old[:, None] * o + a_blk[:, None] * o_blk
        m = m_new
        j0 = j1
    return o / l[:, None], m + np.log(l)
