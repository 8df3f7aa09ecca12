"""Exact attention over FP8 (E4M3) inputs, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the HIP library never
imports this module.

The pages list low-precision FP8 matrix products as a FlashAttention-3
optimisation ("FlashAttention 系列技术详解", section on FlashAttention-3:
hardware-accelerated low-precision GEMM, FP8 doubling tensor-core
throughput).  They fix neither a format nor a scaling contract, so the
readings taken here are:

* the FP8 format is OCP FP8 E4M3 (the "E4M3FN" variant of the OCP 8-bit
  floating point specification): sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals m * 2^-9 in exponent field 0, no infinities,
  and S.1111.111 as NaN;
* each of Q, K, V comes with one float32 dequantisation factor ("descale")
  for the whole tensor: its real value is descale * e4m3(code);
* the operation is the exact attention of those real values, with the same
  scale, masking and LSE as the bf16 path.

So the oracle is the plain definition: decode the codes exactly, multiply by
the descales, and run the float64 attention of ``oracle.attention``.  How
the GPU rounds the probabilities before the P V product is not part of the
definition; the parity tests bound that rounding separately.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_forward, attention_forward_rows


def decode_e4m3(codes) -> np.ndarray:
    """Exact float64 values of OCP E4M3 codes (uint8 array).

    value = (-1)^s * 2^(e - 7) * (1 + m / 8)   for exponent field e in 1..15,
            (-1)^s * 2^-6 * (m / 8)            for e = 0 (subnormals),
    except that e = 15 with m = 7 is NaN (the format has no infinities, so
    the largest finite value is 2^8 * 1.75 = 448).
    """
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError(f"expected uint8 E4M3 codes, got {c.dtype}")
    c = c.astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def dequantize(codes, descale: float) -> np.ndarray:
    """descale * e4m3(code), with descale taken as the float32 value passed."""
    return decode_e4m3(codes) * np.float64(np.float32(descale))


def attention_forward_fp8(q8, k8, v8, descale_q: float, descale_k: float,
                          descale_v: float, scale: float, causal: bool,
                          row_chunk: int | None = None):
    """O and LSE (float64) of exact attention over dequantised E4M3 inputs.

    ``q8``, ``k8``, ``v8`` are uint8 code arrays ``[B, H, N, d]``.
    """
    q = dequantize(q8, descale_q)
    k = dequantize(k8, descale_k)
    v = dequantize(v8, descale_v)
    return attention_forward(q, k, v, scale, causal, row_chunk)


def attention_forward_fp8_rows(q8, k8, v8, descale_q: float, descale_k: float,
                               descale_v: float, scale: float, causal: bool,
                               rows):
    """O and LSE of one head ``[N, d]`` of E4M3 codes for the listed rows."""
    return attention_forward_rows(dequantize(q8, descale_q),
                                  dequantize(k8, descale_k),
                                  dequantize(v8, descale_v), scale, causal, rows)


# ------------------------------------------------------- incoherent processing
# "FlashAttention 系列技术详解", FlashAttention-3 section: before quantising,
# multiply the queries and keys by a random orthogonal matrix, a Hadamard
# transform, which spreads large entries over all coordinates and so lowers
# the quantisation error, at O(d log d) per row.  Reading: the matrix is
# M = diag(signs) H_d / sqrt(d), with H_d the Sylvester Hadamard matrix and
# random signs passed in; (Q M)(K M)^T = Q K^T because M M^T = I, and V is
# not transformed.

def hadamard_matrix(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def incoherent_rotation(x, signs) -> np.ndarray:
    """x M for M = diag(signs) H_d / sqrt(d), over the last axis, float64."""
    x = np.asarray(x, dtype=np.float64)
    s = np.asarray(signs, dtype=np.float64)
    d = x.shape[-1]
    return (x * s) @ hadamard_matrix(d) / np.sqrt(d)


_E4M3_POS = None


def encode_e4m3(x) -> np.ndarray:
    """Nearest E4M3 code to each value (ties to the even code), saturating at
    +-448; finite inputs only.  Written as a nearest-neighbour search over the
    decoded finite codes, the definition of round-to-nearest-even."""
    global _E4M3_POS
    if _E4M3_POS is None:
        _E4M3_POS = decode_e4m3(np.arange(0x7F, dtype=np.uint8))  # codes 0 .. 0x7E, increasing
    v = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(v), _E4M3_POS[-1])
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)


def quantize_e4m3(x, signs=None):
    """Codes and descale of a tensor (rows over the last axis), optionally
    rotated first: y = x M (or x), descale = float32(amax|y| / 448),
    codes = e4m3(y / descale)."""
    y = np.asarray(x, dtype=np.float64) if signs is None else incoherent_rotation(x, signs)
    amax = float(np.max(np.abs(y))) if y.size else 0.0
    descale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    return encode_e4m3(y / descale), descale
