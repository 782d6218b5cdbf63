"""Seeded synthetic attention workloads, shared by the tests, bench.py and smoke().

This module only draws random numbers and casts them; it holds none of the
attention arithmetic, so neither the fp64 oracle nor the HIP path depends on
the other through it.

Recipe: a CPU ``torch.Generator`` seeded per workload draws fp32 N(0, 1)
tensors of shape [B, H, N, d] in the order Q, K, V, dO.  For the sharp-softmax
workload Q and K are multiplied by 8 (a power of two, so exact in bf16 and
independent of whether it is applied before or after the cast).  The GPU
receives the bf16 (round-to-nearest-even) cast; the oracle receives the same
bf16 values widened exactly to fp64.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

__all__ = ["Workload", "WORKLOADS", "draw", "draw_workload", "to_bf16", "bf16_to_f64"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    qk_mult: float = 1.0
    fp32_inputs: bool = False   # the tiny case is drawn and also checked in fp32

    @property
    def scale(self) -> float:
        return 1.0 / (self.d ** 0.5)

    def with_causal(self, causal: bool) -> "Workload":
        return Workload(self.name + ("_causal" if causal else "_full"), self.B, self.H, self.N, self.d,
                        causal, self.seed, self.qk_mult, self.fp32_inputs)


WORKLOADS = {
    "tiny_b1_h1_n128_d64": Workload("tiny_b1_h1_n128_d64", 1, 1, 128, 64, False, 0, fp32_inputs=True),
    "b4_h16_n2048_d128": Workload("b4_h16_n2048_d128", 4, 16, 2048, 128, False, 2),
    "b4_h16_n2048_d128_causal": Workload("b4_h16_n2048_d128_causal", 4, 16, 2048, 128, True, 2),
    "b2_h16_n8192_d128_causal": Workload("b2_h16_n8192_d128_causal", 2, 16, 8192, 128, True, 3),
    "b2_h16_n8192_d128_full": Workload("b2_h16_n8192_d128_full", 2, 16, 8192, 128, False, 3),
    "b4_h8_n4096_d256": Workload("b4_h8_n4096_d256", 4, 8, 4096, 256, False, 4),
    "b2_h8_n4096_d384": Workload("b2_h8_n4096_d384", 2, 8, 4096, 384, False, 6),
    "b2_h8_n4096_d384_causal": Workload("b2_h8_n4096_d384_causal", 2, 8, 4096, 384, True, 6),
    "b1_h32_n16384_d64_causal_sharp": Workload("b1_h32_n16384_d64_causal_sharp", 1, 32, 16384, 64, True, 5,
                                                qk_mult=8.0),
}


def draw(B: int, H: int, N: int, d: int, seed: int, qk_mult: float = 1.0):
    """fp32 CPU tensors (q, k, v, do), drawn in that order from one seeded generator."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    do = torch.randn(shape, generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q = q * qk_mult
        k = k * qk_mult
    return q, k, v, do


def draw_workload(w: Workload):
    return draw(w.B, w.H, w.N, w.d, w.seed, w.qk_mult)


def to_bf16(x: torch.Tensor) -> torch.Tensor:
    """Round-to-nearest-even cast to bfloat16 (torch's float -> bfloat16 rounding)."""
    return x.to(torch.bfloat16)


def bf16_to_f64(x: torch.Tensor):
    """Exact widening of bf16 values to a float64 numpy array."""
    return x.to(torch.float64).numpy()

