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
