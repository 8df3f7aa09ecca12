"""Seeded synthetic inputs shared by the HIP path's tests, the bench and the oracle.

This module draws random numbers and rounds them to bf16; it holds none of
the attention arithmetic.  Both sides of every parity check receive the same
bf16 bit patterns from here: the GPU gets them as a bf16 tensor, the oracle
widens the same bits to float64.

Recipe (the pages' workloads are Q, K, V drawn i.i.d. from N(0, 1), as in the
``torch.randn`` example of "优化的注意力实现", shaped ``[batch, heads, seq,
head_dim]``):

* generator ``numpy.random.Generator(PCG64(seed))``;
* draw order Q, K, V, then dO, each ``standard_normal(shape, float32)``;
* optional Q multiplier (the large-logit stability case uses 8, a power of
  two, so scaling before or after rounding gives the same bits);
* float32 -> bf16 with round-to-nearest-even, once.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16, nearest-even; returns uint16 bit patterns.

    Finite inputs only (the generator never makes NaN or Inf).
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """float32 values of bf16 bit patterns (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def default_scale(d: int) -> float:
    """The float32 value of 1/sqrt(d), returned as a Python float."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_inputs(B: int, H: int, N: int, d: int, seed: int, *,
                q_mult: float = 1.0, with_dout: bool = False) -> dict:
    """Q, K, V (and dO) as uint16 bf16 bit arrays of shape [B, H, N, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal(shape, dtype=np.float32)
        if name == "q" and q_mult != 1.0:
            x = x * np.float32(q_mult)
        out[name] = f32_to_bf16_bits(x)
    if with_dout:
        out["do"] = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return out


@dataclass(frozen=True)
class Workload:
    """A named synthetic workload: shape, masks, passes and variants."""
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: tuple
    backward: bool
    seed: int
    q_mults: tuple = (1.0,)
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return default_scale(self.d)

    def flops_fwd(self, causal: bool) -> float:
        """4 B H N^2 d, halved when causal (the metric's convention)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if causal else f

    def flops_bwd(self, causal: bool) -> float:
        return 2.5 * self.flops_fwd(causal)


WORKLOADS = {
    "c1": Workload("c1", 1, 1, 128, 64, (False,), False, 1000,
                   note="single head, forward only"),
    "c2": Workload("c2", 2, 8, 1024, 64, (True,), False, 2000,
                   note="causal forward, the apxml example's shape"),
    "c3": Workload("c3", 16, 12, 1024, 64, (False, True), False, 3000,
                   q_mults=(1.0, 8.0), note="GPT-2-small attention shape"),
    "c4": Workload("c4", 1, 16, 16384, 128, (True,), False, 4000,
                   note="long-context causal forward"),
    "c5": Workload("c5", 4, 16, 4096, 128, (True,), True, 5000,
                   note="causal forward + backward"),
}
