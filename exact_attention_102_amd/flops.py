"""Work accounting for the benchmark (host logic only).

* pairs: unmasked (query, key) score elements -- N^2 per head, or N(N+1)/2 under
  the causal mask; fully masked tiles are not credited.
* attention_flops: 2 GEMMs in the forward (4 d flop per pair); the backward is
  credited with the 5 GEMMs of the atomic design (10 d per pair) for both designs,
  which is how "Potential algorithmic improvements for backward pass" compares
  them (the 7-GEMM form must run its GEMMs 7/5 faster to tie); the 7-GEMM form
  also reports what it issues, 14 d per pair.
* mfa_op_counts: the per-pair instruction counts of the same page's benchmark
  snippet -- 2D+5 (forward), 3D+5 (dQ kernel), 4D+5 (dK/dV kernel).
"""
from __future__ import annotations


def pairs(N: int, causal: bool, B: int = 1, H: int = 1) -> int:
    per_head = N * (N + 1) // 2 if causal else N * N
    return B * H * per_head


def attention_flops(B: int, H: int, N: int, d: int, causal: bool) -> dict:
    p = pairs(N, causal, B, H)
    return {"pairs": p, "fwd": 4 * d * p, "bwd_effective": 10 * d * p, "bwd_7gemm_issued": 14 * d * p,
            "bwd_5gemm_issued": 10 * d * p}


def mfa_op_counts(N: int, d: int, dispatches: int = 1) -> dict:
    n2 = N * N * dispatches
    return {"forward": (2 * d + 5) * n2, "backward_query": (3 * d + 5) * n2, "backward_key_value": (4 * d + 5) * n2}


def block_size_rule(M: int, d: int) -> int:
    """ceil(M / 4d): rows per block so that q, k, v and o blocks of width d fill an on-chip memory of M
    elements ("ELI5: FlashAttention", step 1 of the walk-through)."""
    return -(-M // (4 * d))


def d_spectrum(limit: int = 384) -> list:
    """Head dimensions of the D sweep in "Potential algorithmic improvements for backward pass": step 4 below
    96, step 8 below 160, step 16 below 256, step 32 below 384 (42 values up to 384)."""
    out, d = [], 0
    for bound, step in ((96, 4), (160, 8), (256, 16), (limit, 32)):
        while d < bound:
            d += step
            out.append(d)
    return out
