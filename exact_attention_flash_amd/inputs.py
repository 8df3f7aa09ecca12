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

FP8 variant (``make_inputs_fp8``): the same float32 draws, each tensor
divided by its own amax / 448 and rounded once to OCP E4M3 (nearest-even,
saturating); the descale amax / 448 travels with the codes.
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


# ---------------------------------------------------------------- fp8 inputs
E4M3_MAX = 448.0  # largest finite OCP E4M3 value, 1.75 * 2^8


def f32_to_e4m3_bits(x) -> np.ndarray:
    """Round values to OCP FP8 E4M3 ("E4M3FN"), nearest-even; returns uint8 codes.

    Saturating: magnitudes above 448 give 448.  Finite inputs only.  Layout
    of a code: sign bit, 4 exponent bits (bias 7), 3 mantissa bits; exponent
    field 0 holds the subnormals m * 2^-9.
    """
    a = np.asarray(x, dtype=np.float64)
    sign = np.signbit(a).astype(np.uint8) << np.uint8(7)
    mag = np.minimum(np.abs(a), E4M3_MAX)
    frac, ex = np.frexp(mag)                 # mag = frac * 2^ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1              # mag = (2 frac) * 2^e
    normal = mag >= 2.0 ** -6  # (zero has e = -1 from frexp, so test the value)
    # normal range: 3 fraction bits of 2 frac in [1, 2); a carry out of the
    # fraction moves to the next exponent (never past 448, which is a code)
    q = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    code_n = ((e + 7) << 3) | q
    # subnormal range: multiples of 2^-9; 8 * 2^-9 is the smallest normal,
    # whose code is 8 as well
    code_s = np.rint(mag * 512.0).astype(np.int64)
    code = np.where(normal, code_n, code_s)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_descale(x) -> float:
    """Per-tensor dequantisation factor amax / 448, as a float32 value.

    The tensor is stored as codes of x / descale, which puts its largest
    magnitude at the top of the E4M3 range (amax scaling).  An all-zero
    tensor gets descale 1.
    """
    amax = float(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else 0.0
    return float(np.float32(amax / E4M3_MAX)) if amax > 0 else 1.0


def make_inputs_fp8(B: int, H: int, N: int, d: int, seed: int, *,
                    q_mult: float = 1.0) -> dict:
    """Q, K, V as uint8 E4M3 codes of shape [B, H, N, d] with their descales.

    The same float32 draws as ``make_inputs`` (same generator, order and Q
    multiplier); each tensor then gets its own amax descale and is rounded
    once to E4M3.  The real value of a code c is descale * e4m3(c).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal(shape, dtype=np.float32)
        if name == "q" and q_mult != 1.0:
            x = x * np.float32(q_mult)
        ds = e4m3_descale(x)
        out[name] = f32_to_e4m3_bits(x.astype(np.float64) / ds)
        out["descale_" + name] = ds
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
